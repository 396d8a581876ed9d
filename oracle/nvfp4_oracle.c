/*
 * NVFP4 paged KV cache -- CPU ORACLE.  TEST INFRASTRUCTURE ONLY.
 *
 * Plain, scalar, float64 statement of what the NVFP4 KV-cache hot path
 * computes.  Only the test suite, the smoke check and the bench's CPU-baseline
 * leg load this file; the HIP library never includes, links or calls it, and
 * it shares no code, header, table or helper with that library.
 *
 * Sources (web pages; cited by title and section):
 *   [MW]  grer.cn blog, "NVFP4 KV cache and the memory wall"
 *         §1 memory accounting, §2 two-level scaling (value list + stdlib
 *         experiment), §3 the three data flows in the serving engine.
 *   [NV]  nmedialink.com, "NVIDIA NVFP4: LLM memory doubled, inference 3x"
 *         section on the KV-cache quantize/dequantize flow (Fig. 3).
 *   [TC]  cloud.tencent.com.cn, "NVFP4: breaking the memory wall of GPU
 *         inference", section "E2M1 encoding and two-level scaling".
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes):
 *   R1 ties go to the even code (E2M1) / even byte (E4M3); the page's own
 *      experiment breaks ties toward the more negative list entry, which
 *      makes no difference on its Gaussian data (ties have measure zero).
 *   R2 block scale = E4M3 value nearest to amax/(6*g) (the page's script keeps
 *      it unrounded and has no g); saturates at 448, values below the E4M3
 *      grid's half-step round to 0.
 *   R3 codes saturate at magnitude 6 (code 7).
 *   R4 E4M3 is OCP E4M3FN: bias 7, subnormals m*2^-9, max 448, no infinity.
 *   R5 the sign bit of a code is the sign bit of the input (so -0.0 and small
 *      negatives that round to 0 give code 0x8).
 *   R6 blocks are 16 consecutive values along head_dim of one (token, head).
 *   R7 low nibble = even element.
 *   R8 a zero scale (amax == 0 or amax/(6g) rounding to 0) gives scale byte 0
 *      and magnitude code 0 for every element.
 *   R9 MXFP4 (the comparison format) follows the OCP MX v1.0 definition; see
 *      the MXFP4 section below.
 *   R10 the Hadamard rotation of K (and Q) is the 128-point Sylvester matrix
 *      with power-of-two scales; see the Hadamard section below.
 *   R11 extend attention in FP8 arithmetic rounds Q (per row, power-of-two
 *      scale) and the softmax weights (relative to the ceiling of the row's
 *      maximum base-2 logit, 2^8 headroom) to E4M3; see that section below.
 *
 * Exactness of the float64 quotients used below.  Inputs are float32 (24-bit
 * significands), g is float32, block scales are E4M3 (4-bit significands) and
 * every rounding boundary (a midpoint between two adjacent grid values) has at
 * most 5 significant bits.  A boundary times the divisor therefore has at most
 * 5 + 24 + 2 = 31 significant bits, while the dividend has 24 (or 30 for a
 * dequantized value), so a dividend that is not exactly on a boundary is at
 * least 2^-32 (relative) away from it -- far more than the 2^-53 error of one
 * correctly rounded float64 division.  Exact ties divide exactly.  Hence
 * rounding the float64 quotient gives the same grid point as rounding the
 * exact real quotient.  Products bs*g (28 bits) and e2m1*bs*g (30 bits) are
 * exact in float64.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* E2M1 value of a 4-bit code: bit 3 sign, bits 2..1 exponent (bias 1),
 * bit 0 mantissa; exponent 0 is subnormal (mantissa * 0.5).  [TC] encoding
 * section (1 sign, 2 exponent, 1 mantissa bit); the resulting magnitudes are
 * the list in [MW] §2. */
double nvfp4o_e2m1_value(int code) {
  int e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return (code & 8) ? -mag : mag;
}

/* OCP E4M3FN value of a byte (reading R4): bit 7 sign, bits 6..3 exponent
 * (bias 7), bits 2..0 mantissa; exponent 0 subnormal m/8 * 2^-6; 0x7F/0xFF NaN.
 * [MW] §2 and [TC]: the per-16 block scale is FP8 E4M3. */
double nvfp4o_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest non-negative finite E4M3 value to r >= 0; ties to the even byte;
 * everything above 448 goes to 448 (readings R2, R4).  Brute force over the
 * 127 finite non-negative bytes. */
int nvfp4o_e4m3_encode(double r) {
  if (r >= 448.0) return 0x7E; /* saturation: 448 is the nearest finite value */
  int best = 0;
  double bestd = fabs(r - 0.0);
  for (int b = 1; b <= 0x7E; ++b) {
    double d = fabs(r - nvfp4o_e4m3_value(b));
    if (d < bestd || (d == bestd && (b & 1) == 0 && (best & 1) == 1)) {
      best = b;
      bestd = d;
    }
  }
  return best;
}

/* Nearest E2M1 magnitude code (0..7) to y >= 0; ties to the even code;
 * y above 6 goes to code 7 (readings R1, R3).  Brute force over 8 values. */
int nvfp4o_e2m1_encode(double y) {
  if (y >= 6.0) return 7; /* saturation: 6 is the nearest value */
  int best = 0;
  double bestd = fabs(y);
  for (int c = 1; c < 8; ++c) {
    double d = fabs(y - nvfp4o_e2m1_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* ----------------------------------------------------------- quantization */

/* Two-level NVFP4 quantization of rows of 128 values (one row = one token of
 * one KV head) with FP32 global scale g ([MW] §2: 16 consecutive values share
 * one E4M3 scale, the whole tensor shares one FP32 scale; [TC] same).
 *   codes : n_rows x 64 bytes, byte j = code(2j) | code(2j+1) << 4   (R7)
 *   scales: n_rows x 8 bytes, byte b = E4M3 scale of values 16b..16b+15 (R6)
 * Per block: amax = max|x|, bs = E4M3(amax/(6g)) (R2), each code = sign(x) |
 * E2M1(|x|/(bs*g)) (R1, R3, R5), zero scale -> magnitude 0 (R8). */
/* One 16-value block: its E4M3 scale byte and its 16 codes, ORed into the 8
 * code bytes cb (which start at zero). */
static void quantize_block16(const float* xb, double gd, uint8_t* cb, uint8_t* sb) {
  double amax = 0.0;
  for (int i = 0; i < 16; ++i) {
    double a = fabs((double)xb[i]);
    if (a > amax) amax = a;
  }
  int sbyte = nvfp4o_e4m3_encode(amax / (6.0 * gd));
  double bs = nvfp4o_e4m3_value(sbyte);
  *sb = (uint8_t)sbyte;
  for (int i = 0; i < 16; ++i) {
    double v = (double)xb[i];
    int mag = (bs == 0.0) ? 0 : nvfp4o_e2m1_encode(fabs(v) / (bs * gd));
    int code = (signbit(v) ? 8 : 0) | mag;
    cb[i / 2] |= (uint8_t)(code << (4 * (i & 1)));
  }
}

void nvfp4o_quantize_rows(const float* x, int64_t n_rows, float g, uint8_t* codes, uint8_t* scales) {
  const double gd = (double)g;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    memset(codes + r * 64, 0, 64);
    for (int b = 0; b < 8; ++b) quantize_block16(x + r * 128 + 16 * b, gd, codes + r * 64 + 8 * b, scales + r * 8 + b);
  }
}

/* x_hat = E2M1(code) * E4M3(scale) * g, the dequantized value ([MW] §2 and
 * §3: the block scale and the tensor-wide FP32 scale multiply the 4-bit
 * value).  Exact in float64. */
void nvfp4o_dequantize_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, float g, double* out) {
  for (int64_t r = 0; r < n_rows; ++r)
    for (int d = 0; d < 128; ++d) {
      int code = (codes[r * 64 + d / 2] >> (4 * (d & 1))) & 15;
      out[r * 128 + d] = nvfp4o_e2m1_value(code) * nvfp4o_e4m3_value(scales[r * 8 + d / 16]) * (double)g;
    }
}

/* ------------------------------------------------------------- page layout
 * A page holds 16 token slots; slot s -> page p = s/16, offset o = s%16.
 * Per (page, kv head) each plane holds a 1 KiB code tile and a 128 B scale
 * tile (64 + 8 bytes per token and head: 9/16 byte per value, [MW] §1).
 *   K codes : tile byte o*64 + d/2                                   nibble d%2
 *   K scales: tile byte o*8 + d/16
 *   V codes : tile byte (o/4)*256 + (d/8)*16 + ((o/2)%2)*8 + (d%2)*4 + (d%8)/2
 *                                                                    nibble o%2
 *   V scales: tile byte (d/16)*16 + o
 * (nibble 0 = low).  A V code byte holds one dimension of two neighbouring
 * slots (o even in the low nibble, o+1 in the high one).  The pages fix no
 * in-page arrangement; this one is the library's.  Tile (p, h) starts at
 * (p*H + h)*1024 in a code plane and at (p*H + h)*128 in a scale plane. */
static int64_t k_code_byte(int64_t p, int h, int H, int o, int d) { return (p * H + h) * 1024 + o * 64 + d / 2; }
static int64_t k_scale_byte(int64_t p, int h, int H, int o, int b) { return (p * H + h) * 128 + o * 8 + b; }
static int64_t v_code_byte(int64_t p, int h, int H, int o, int d) {
  return (p * H + h) * 1024 + (o / 4) * 256 + (d / 8) * 16 + ((o / 2) % 2) * 8 + (d % 2) * 4 + (d % 8) / 2;
}
static int64_t v_scale_byte(int64_t p, int h, int H, int o, int b) { return (p * H + h) * 128 + b * 16 + o; }

/* Byte and nibble shift (0 or 4) of dimension d of slot offset o in the
 * tile (p, h) of an NVFP4 code plane. */
static int64_t code_at(int is_v, int64_t p, int h, int H, int o, int d, int* shift) {
  *shift = 4 * (is_v ? (o & 1) : (d & 1));
  return is_v ? v_code_byte(p, h, H, o, d) : k_code_byte(p, h, H, o, d);
}

/* Write quantized rows (row index t*H + h) into the planes at slot_mapping[t];
 * negative slots are skipped. is_v selects the V layout. */
void nvfp4o_scatter_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_tokens, int H, const int32_t* slot_mapping,
                         int is_v, uint8_t* code_plane, uint8_t* scale_plane) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t p = s / 16;
    int o = (int)(s % 16);
    for (int h = 0; h < H; ++h) {
      const uint8_t* cr = codes + (t * H + h) * 64;
      const uint8_t* sr = scales + (t * H + h) * 8;
      for (int d = 0; d < 128; ++d) {
        int code = (cr[d / 2] >> (4 * (d & 1))) & 15;
        int sh;
        int64_t at = code_at(is_v, p, h, H, o, d, &sh);
        code_plane[at] = (uint8_t)((code_plane[at] & ~(15 << sh)) | (code << sh));
      }
      for (int b = 0; b < 8; ++b)
        scale_plane[is_v ? v_scale_byte(p, h, H, o, b) : k_scale_byte(p, h, H, o, b)] = sr[b];
    }
  }
}

/* Dequantized value of dimension d of (slot s, head h) read from the planes. */
static double plane_value(const uint8_t* code_plane, const uint8_t* scale_plane, int is_v, int64_t s, int h, int H, int d,
                          double g) {
  int64_t p = s / 16;
  int o = (int)(s % 16);
  int sh;
  int64_t at = code_at(is_v, p, h, H, o, d, &sh);
  int code = (code_plane[at] >> sh) & 15;
  int sb = scale_plane[is_v ? v_scale_byte(p, h, H, o, d / 16) : k_scale_byte(p, h, H, o, d / 16)];
  return nvfp4o_e2m1_value(code) * nvfp4o_e4m3_value(sb) * g;
}

/* Read logical rows back out of the planes (codes and scale bytes), for the
 * layout tests. */
void nvfp4o_gather_rows(const uint8_t* code_plane, const uint8_t* scale_plane, int64_t n_tokens, int H,
                        const int32_t* slot_mapping, int is_v, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    int64_t p = s / 16;
    int o = (int)(s % 16);
    for (int h = 0; h < H; ++h) {
      uint8_t* cr = codes + (t * H + h) * 64;
      memset(cr, 0, 64);
      for (int d = 0; d < 128; ++d) {
        int sh;
        int64_t at = code_at(is_v, p, h, H, o, d, &sh);
        int code = (code_plane[at] >> sh) & 15;
        cr[d / 2] |= (uint8_t)(code << (4 * (d & 1)));
      }
      for (int b = 0; b < 8; ++b)
        scales[(t * H + h) * 8 + b] = scale_plane[is_v ? v_scale_byte(p, h, H, o, b) : k_scale_byte(p, h, H, o, b)];
    }
  }
}

/* ------------------------------------------------------ decode attention
 * One decode step over the paged NVFP4 cache ([MW] §3, third data flow: the
 * decode kernel dequantizes K/V where it reads them; [NV] KV-cache primer:
 * the new query attends over every cached K/V).  For each selected query row
 * (b, qh), with kv head h = qh / (Hq/Hkv) (grouped-query heads, [MW] §1):
 *   s_t = sm_scale * sum_d q[d] * K_hat[t][d]   for t < seq_lens[b]
 *   p   = softmax(s)                            (float64, max-subtracted)
 *   o   = sum_t p_t * V_hat[t]
 * token t lives in slot block_table[b*bt_stride + t/16]*16 + t%16.  An empty
 * sequence gives o = 0.  rows[i] = b*Hq + qh; out is n_rows x 128 float64. */
typedef double (*plane_value_fn)(const uint8_t* code_plane, const uint8_t* scale_plane, int is_v, int64_t s, int h,
                                 int H, int d, double g);

static void decode_attention_with(plane_value_fn value, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                                  const uint8_t* vs, int Hkv, float g_k, float g_v, const float* q, int Hq,
                                  const int32_t* block_table, int bt_stride, const int32_t* seq_lens, float sm_scale,
                                  const int64_t* rows, int64_t n_rows, double* out) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t b = rows[i] / Hq;
    int qh = (int)(rows[i] % Hq);
    int h = qh / G;
    int64_t n = seq_lens[b];
    const float* qr = q + rows[i] * 128;
    double* o = out + i * 128;
    for (int d = 0; d < 128; ++d) o[d] = 0.0;
    if (n <= 0) continue;
    double* s = (double*)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      int64_t slot = (int64_t)block_table[b * bt_stride + t / 16] * 16 + t % 16;
      double acc = 0.0;
      for (int d = 0; d < 128; ++d) acc += (double)qr[d] * value(kc, ks, 0, slot, h, Hkv, d, g_k);
      s[t] = (double)sm_scale * acc;
      if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      int64_t slot = (int64_t)block_table[b * bt_stride + t / 16] * 16 + t % 16;
      double pt = exp(s[t] - m);
      l += pt;
      for (int d = 0; d < 128; ++d) o[d] += pt * value(vc, vs, 1, slot, h, Hkv, d, g_v);
    }
    free(s);
    for (int d = 0; d < 128; ++d) o[d] /= l;
  }
}

void nvfp4o_decode_attention(const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int Hkv, float g_k,
                             float g_v, const float* q, int Hq, const int32_t* block_table, int bt_stride,
                             const int32_t* seq_lens, float sm_scale, const int64_t* rows, int64_t n_rows, double* out) {
  decode_attention_with(plane_value, kc, ks, vc, vs, Hkv, g_k, g_v, q, Hq, block_table, bt_stride, seq_lens, sm_scale,
                        rows, n_rows, out);
}

/* ----------------------------------------------------- FP8 workspace dequant
 * Extend / chunked-prefill flow ([MW] §3 second data flow; [NV] Fig. 3: the
 * NVFP4 cache is dequantized to FP8 before the attention that consumes it).
 * For extend sequence i and cached token t < prefix_lens[i]:
 *   ws[(ws_offsets[i] + t)*Hkv*128 + h*128 + d] =
 *       sign(x_hat) | E4M3(|x_hat| / ws_scale)       x_hat = E2M1*bs*g
 * E4M3 rounding as the block scale (nearest, ties to even, saturate at 448);
 * the sign bit follows x_hat, so -0.0 and tiny negatives give 0x80. */
void nvfp4o_fp8_workspace(const uint8_t* code_plane, const uint8_t* scale_plane, int is_v, int Hkv, float g,
                          const int32_t* block_table, int bt_stride, int num_seqs, const int32_t* prefix_lens,
                          const int32_t* ws_offsets, float ws_scale, uint8_t* ws) {
  for (int i = 0; i < num_seqs; ++i) {
    int64_t n = prefix_lens[i];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
      int64_t slot = (int64_t)block_table[(int64_t)i * bt_stride + t / 16] * 16 + t % 16;
      for (int h = 0; h < Hkv; ++h)
        for (int d = 0; d < 128; ++d) {
          double xh = plane_value(code_plane, scale_plane, is_v, slot, h, Hkv, d, (double)g);
          int byte = nvfp4o_e4m3_encode(fabs(xh) / (double)ws_scale);
          if (signbit(xh)) byte |= 0x80;
          ws[((int64_t)ws_offsets[i] + t) * Hkv * 128 + h * 128 + d] = (uint8_t)byte;
        }
    }
  }
}

/* ------------------------------------------------ FP8 rows of a new chunk
 * [MW] §3, first and second data flows: the K/V of the tokens being
 * prefilled or extended take part in attention as FP8 (only the cached prefix
 * goes through the NVFP4 -> FP8 workspace).  Reading: they are stored into
 * workspace rows with the workspace's own per-tensor scale, by the same
 * rounding as above (E4M3 nearest to |x| / ws_scale, ties to even, saturating
 * at 448; sign bit of x).  x is n_tokens x stride floats, token t's head h
 * at x[t*stride + h*128]; rows[t] < 0 skips token t. */
void nvfp4o_fp8_quantize_rows(const float* x, int64_t n_tokens, int64_t stride, int Hkv, const int32_t* rows,
                              float ws_scale, uint8_t* ws) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tokens; ++t) {
    if (rows[t] < 0) continue;
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < 128; ++d) {
        double xv = (double)x[t * stride + h * 128 + d];
        int byte = nvfp4o_e4m3_encode(fabs(xv) / (double)ws_scale);
        if (signbit(xv)) byte |= 0x80;
        ws[((int64_t)rows[t] * Hkv + h) * 128 + d] = (uint8_t)byte;
      }
  }
}

/* ------------------------------------------ extend attention over FP8 rows
 * [MW] §3 second data flow (chunked prefill / extend): the chunk's queries
 * attend over the cached prefix, read from the FP8 workspace, and over the
 * chunk itself, causally as in prefill ([MW] §3 first data flow; the chunk's
 * K/V are FP8 rows after the prefix, see nvfp4o_fp8_quantize_rows).
 * Sequence i: prefix P_i = prefix_lens[i], chunk C_i = q_offsets[i+1] -
 * q_offsets[i]; its K/V rows are ws_offsets[i] + t, t < P_i + C_i.  Query
 * token j < C_i (row q_offsets[i] + j of q) sits at position P_i + j and sees
 * keys t <= P_i + j.  For query head qh, kv head h = qh / (Hq/Hkv) ([MW] §1):
 *   s_t = sm_scale * sum_d q[d] * E4M3(ws_k[row_t][h][d]) * k_ws_scale
 *   o   = sum_t softmax(s)_t * E4M3(ws_v[row_t][h][d]) * v_ws_scale
 * in float64.  rows[r] = (query row) * Hq + qh selects the outputs computed;
 * out is n_rows x 128. */
void nvfp4o_extend_attention(const uint8_t* ws_k, const uint8_t* ws_v, int Hkv, float k_ws_scale, float v_ws_scale,
                             const float* q, int Hq, int num_seqs, const int32_t* q_offsets,
                             const int32_t* ws_offsets, const int32_t* prefix_lens, float sm_scale,
                             const int64_t* rows, int64_t n_rows, double* out) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t qrow = rows[r] / Hq;
    const int qh = (int)(rows[r] % Hq), h = qh / G;
    int i = 0;
    while (i < num_seqs - 1 && q_offsets[i + 1] <= qrow) ++i; /* the sequence holding this query row */
    const int64_t j = qrow - q_offsets[i];
    const int64_t n = (int64_t)prefix_lens[i] + j + 1; /* keys 0 .. P_i + j */
    const float* qv = q + rows[r] * 128;
    double* o = out + r * 128;
    double* s = (double*)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      const uint8_t* kr = ws_k + (((int64_t)ws_offsets[i] + t) * Hkv + h) * 128;
      double acc = 0.0;
      for (int d = 0; d < 128; ++d) acc += (double)qv[d] * (nvfp4o_e4m3_value(kr[d]) * (double)k_ws_scale);
      s[t] = (double)sm_scale * acc;
      if (s[t] > m) m = s[t];
    }
    for (int d = 0; d < 128; ++d) o[d] = 0.0;
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      const uint8_t* vr = ws_v + (((int64_t)ws_offsets[i] + t) * Hkv + h) * 128;
      const double pt = exp(s[t] - m);
      l += pt;
      for (int d = 0; d < 128; ++d) o[d] += pt * (nvfp4o_e4m3_value(vr[d]) * (double)v_ws_scale);
    }
    free(s);
    for (int d = 0; d < 128; ++d) o[d] /= l;
  }
}

/* ------------------------------- extend attention in FP8 arithmetic
 * [MW] §3: extend attention consumes the FP8 workspace directly.  On
 * hardware whose matrix cores take E4M3 operands, Q and the softmax weights
 * enter them as E4M3 too; the pages do not spell that arithmetic out, so this
 * is reading R11 (the plainest FP8 statement of the same attention):
 *   c    = float32(sm_scale * k_ws_scale * log2 e);   u_d = float32(q_d * c)
 *   Q8_d = E4M3(u_d * 2^-E)   E = the smallest integer with max_d |u_d| <= 448 * 2^E
 *                             (0 for a zero row); nearest, ties to even (R1, R4);
 *   x_t  = 2^E * sum_d Q8_d * E4M3(k_td)
 *   M    = ceil(max_t x_t);   W_t = E4M3(2^(x_t - M + h))   (<= 256)
 *                             h = 8 for |M| < 2^27, else 0 (float32 holds M - 8
 *                             exactly only below 2^27);
 *   o_d  = v_ws_scale * sum_t W_t E4M3(v_td) / sum_t W_t.
 * Keys and sequences as in nvfp4o_extend_attention.  The logits are exact in
 * float64 (E4M3 products have at most 8 significant bits over 36 binades;
 * 128 of them fit 53 bits), and so is u_d (a product of two float32 values,
 * rounded once to float32).
 *
 * tol[r] bounds |o_GPU - o| for one row of a kernel that computes the same
 * thing with float32 logits and an integer running maximum (it rescales by
 * exact powers of two), on FP8 matrix cores whose dot products of up to 64
 * terms are within 2^-11 of their largest product.  It sums:
 *   - accumulation: 2^-10 * sum_t W_t * vmax_t over the numerator, 2^-10 * L
 *     over the sum L = sum_t W_t (vmax_t = max_d |v_td| in output units);
 *   - rounding flips: a weight whose exact value lies within the relative
 *     error e_t of the kernel's 2^(x - m + 8) from an E4M3 midpoint may take
 *     the neighbouring value; e_t = ln2 * (2^E * (2^-10 * max_d |Q8_d k_td|
 *     + 2^-23 * sum_d |Q8_d k_td|) + 2^-22 * |x_t| + 2^-22) + 2^-21;
 *   - small weights (below 2^-5 at M): rounded at another power-of-two
 *     scale, within 2^-8 of this one;
 * each weight change times vmax_t in the numerator and alone in L, then
 * |dN| / (L - |dL|) + max_d |o_d| * |dL| / (L - |dL|), plus 2^-20 * max |o|.
 * rows[r] = (query row) * Hq + qh; out is n_rows x 128, tol n_rows. */
static int e4m3_code_of(double y) { return nvfp4o_e4m3_encode(y); }

void nvfp4o_extend_attention_fp8(const uint8_t* ws_k, const uint8_t* ws_v, int Hkv, float k_ws_scale,
                                 float v_ws_scale, const float* q, int Hq, int num_seqs, const int32_t* q_offsets,
                                 const int32_t* ws_offsets, const int32_t* prefix_lens, float sm_scale,
                                 const int64_t* rows, int64_t n_rows, double* out, double* tol) {
  const int G = Hq / Hkv;
  const float c = (float)((double)sm_scale * (double)k_ws_scale * 1.4426950408889634);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t qrow = rows[r] / Hq;
    const int qh = (int)(rows[r] % Hq), h = qh / G;
    int i = 0;
    while (i < num_seqs - 1 && q_offsets[i + 1] <= qrow) ++i;
    const int64_t j = qrow - q_offsets[i];
    const int64_t n = (int64_t)prefix_lens[i] + j + 1;
    const float* qv = q + rows[r] * 128;
    double* o = out + r * 128;
    /* Q8 */
    double u[128], amax = 0.0;
    for (int d = 0; d < 128; ++d) {
      u[d] = (double)(float)((double)qv[d] * (double)c);
      amax = fmax(amax, fabs(u[d]));
    }
    int E = 0;
    if (amax > 0.0) {
      E = -200;
      while (amax > 448.0 * ldexp(1.0, E)) ++E;
    }
    double q8[128];
    for (int d = 0; d < 128; ++d) {
      const double a = ldexp(u[d], -E);
      const double mag = nvfp4o_e4m3_value(e4m3_code_of(fabs(a)));
      q8[d] = signbit(a) ? -mag : mag;
    }
    const double cs = ldexp(1.0, E);
    double* x = (double*)malloc((size_t)n * sizeof(double));
    double* ex = (double*)malloc((size_t)n * sizeof(double));
    double xmax = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      const uint8_t* kr = ws_k + (((int64_t)ws_offsets[i] + t) * Hkv + h) * 128;
      double sdot = 0.0, pmax = 0.0, psum = 0.0;
      for (int d = 0; d < 128; ++d) {
        const double pr = q8[d] * nvfp4o_e4m3_value(kr[d]);
        sdot += pr;
        pmax = fmax(pmax, fabs(pr));
        psum += fabs(pr);
      }
      x[t] = sdot * cs;
      ex[t] = 0.6931471805599453 * (fabs(cs) * (ldexp(pmax, -10) + ldexp(psum, -23)) + ldexp(fabs(x[t]), -22) + ldexp(1.0, -22)) +
              ldexp(1.0, -21);
      if (x[t] > xmax) xmax = x[t];
    }
    const double M = ceil(xmax);
    double l = 0.0;
    for (int d = 0; d < 128; ++d) o[d] = 0.0;
    double wsum_v = 0.0, flip_l = 0.0, flip_n = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      const uint8_t* vr = ws_v + (((int64_t)ws_offsets[i] + t) * Hkv + h) * 128;
      const double y = exp2(x[t] - M + (fabs(M) < 134217728.0 ? 8.0 : 0.0));
      const int code = e4m3_code_of(y);
      const double w = nvfp4o_e4m3_value(code);
      double vmax = 0.0;
      for (int d = 0; d < 128; ++d) {
        const double v = nvfp4o_e4m3_value(vr[d]) * (double)v_ws_scale;
        o[d] += w * v;
        vmax = fmax(vmax, fabs(v));
      }
      l += w;
      wsum_v += w * vmax;
      /* a flip to a neighbouring code, or a small weight rounded at another scale */
      double dw = 0.0;
      if (y < 0.03125) dw = ldexp(1.0, -8);
      const double lo = code > 0 ? 0.5 * (nvfp4o_e4m3_value(code - 1) + w) : -1.0;
      const double hi = code < 0x7E ? 0.5 * (w + nvfp4o_e4m3_value(code + 1)) : INFINITY;
      if (y * (1.0 - ex[t]) <= lo || y * (1.0 + ex[t]) >= hi) {
        const double step = fmax(code > 0 ? w - nvfp4o_e4m3_value(code - 1) : 0.0,
                                 code < 0x7E ? nvfp4o_e4m3_value(code + 1) - w : 0.0);
        dw = fmax(dw, step);
      }
      flip_l += dw;
      flip_n += dw * vmax;
    }
    free(x);
    free(ex);
    double omax = 0.0;
    for (int d = 0; d < 128; ++d) {
      o[d] = l > 0.0 ? o[d] / l : 0.0;
      omax = fmax(omax, fabs(o[d]));
    }
    const double dn = ldexp(wsum_v, -10) + flip_n;
    const double dl = ldexp(l, -10) + flip_l;
    tol[r] = (l > dl) ? (dn + omax * dl) / (l - dl) + ldexp(omax, -20) : INFINITY;
  }
}

/* ------------------------------------------------------------------ MXFP4
 * The 4-bit format the pages compare NVFP4 against ([NV] accuracy section and
 * Fig. 6: NVFP4 KV caches score higher than MXFP4 ones, credited to the finer
 * blocks and the E4M3 scales; [TC] "E2M1 encoding and two-level scaling":
 * MXFP4 shares one scale among 32 values where NVFP4 uses 16).  The pages
 * define no more of it; the rest is the published OCP Microscaling (MX) v1.0
 * definition of MXFP4 (reading R9):
 *   - E2M1 elements, 32 consecutive values along head_dim per block (so a
 *     128-value row has 4 blocks), no tensor-wide scale;
 *   - the block scale is a power of two X = 2^(byte - 127) stored as an E8M0
 *     byte (0xFF is NaN);
 *   - X = 2^(floor(log2 amax) - 2), where 2 is the exponent of the largest
 *     E2M1 value (6 = 1.5 * 2^2), clamped to 2^-127 .. 2^127; amax = 0 takes
 *     2^-127 (byte 0);
 *   - element = sign(x) | E2M1 nearest to |x| / X, ties to the even code and
 *     saturating at 6 (R1, R3, R5, R7 as for NVFP4).
 * |x| / X is exact in float64 (a power of two), so the rounding is exact. */
double nvfp4o_e8m0_value(int byte) { return byte == 255 ? NAN : ldexp(1.0, byte - 127); }

/* E8M0 byte of the MXFP4 block scale for a block maximum amax >= 0. */
int nvfp4o_e8m0_scale_for(double amax) {
  if (!(amax > 0.0)) return 0;
  int e;
  (void)frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
  int x = (e - 1) - 2;
  if (x < -127) x = -127;
  if (x > 127) x = 127;
  return x + 127;
}

/* Rows of 128 values to MXFP4: codes n_rows x 64 bytes (byte j = code(2j) |
 * code(2j+1) << 4), scales n_rows x 4 E8M0 bytes (byte b: values 32b..32b+31). */
void nvfp4o_mx_quantize_rows(const float* x, int64_t n_rows, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const float* xr = x + r * 128;
    uint8_t* cr = codes + r * 64;
    memset(cr, 0, 64);
    for (int b = 0; b < 4; ++b) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        double a = fabs((double)xr[32 * b + i]);
        if (a > amax) amax = a;
      }
      int sb = nvfp4o_e8m0_scale_for(amax);
      double X = nvfp4o_e8m0_value(sb);
      scales[r * 4 + b] = (uint8_t)sb;
      for (int i = 0; i < 32; ++i) {
        int d = 32 * b + i;
        double v = (double)xr[d];
        int code = (signbit(v) ? 8 : 0) | nvfp4o_e2m1_encode(fabs(v) / X);
        cr[d / 2] |= (uint8_t)(code << (4 * (d & 1)));
      }
    }
  }
}

/* x_hat = E2M1(code) * 2^(scale byte - 127), exact in float64. */
void nvfp4o_mx_dequantize_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, double* out) {
  for (int64_t r = 0; r < n_rows; ++r)
    for (int d = 0; d < 128; ++d) {
      int code = (codes[r * 64 + d / 2] >> (4 * (d & 1))) & 15;
      out[r * 128 + d] = nvfp4o_e2m1_value(code) * nvfp4o_e8m0_value(scales[r * 4 + d / 32]);
    }
}

/* MXFP4 pages: K codes as the NVFP4 K codes; V codes keep each slot's nibbles
 * in bytes of its own (a V byte's two values share one E8M0 scale only if they
 * are one slot's):
 *   V codes : tile byte (o/4)*256 + (d/8)*16 + (o%4)*4 + (d%8)/2   nibble d%2
 * A scale tile is 64 bytes (4 per token):
 *   K scales: tile byte o*4 + d/32         V scales: tile byte (d/32)*16 + o
 * Tile (p, h) starts at (p*H + h)*64 in a scale plane: 68 bytes per (token,
 * kv head) per tensor, 17/32 byte per value. */
static int64_t mx_scale_byte(int is_v, int64_t p, int h, int H, int o, int b) {
  return (p * H + h) * 64 + (is_v ? b * 16 + o : o * 4 + b);
}
static int64_t mx_code_byte(int is_v, int64_t p, int h, int H, int o, int d) {
  return is_v ? (p * H + h) * 1024 + (o / 4) * 256 + (d / 8) * 16 + (o % 4) * 4 + (d % 8) / 2
              : k_code_byte(p, h, H, o, d);
}

void nvfp4o_mx_scatter_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_tokens, int H,
                            const int32_t* slot_mapping, int is_v, uint8_t* code_plane, uint8_t* scale_plane) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t p = s / 16;
    int o = (int)(s % 16);
    for (int h = 0; h < H; ++h) {
      const uint8_t* cr = codes + (t * H + h) * 64;
      for (int d = 0; d < 128; ++d) {
        int code = (cr[d / 2] >> (4 * (d & 1))) & 15;
        int64_t at = mx_code_byte(is_v, p, h, H, o, d);
        int sh = 4 * (d & 1);
        code_plane[at] = (uint8_t)((code_plane[at] & ~(15 << sh)) | (code << sh));
      }
      for (int b = 0; b < 4; ++b) scale_plane[mx_scale_byte(is_v, p, h, H, o, b)] = scales[(t * H + h) * 4 + b];
    }
  }
}

void nvfp4o_mx_gather_rows(const uint8_t* code_plane, const uint8_t* scale_plane, int64_t n_tokens, int H,
                           const int32_t* slot_mapping, int is_v, uint8_t* codes, uint8_t* scales) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    int64_t p = s / 16;
    int o = (int)(s % 16);
    for (int h = 0; h < H; ++h) {
      uint8_t* cr = codes + (t * H + h) * 64;
      memset(cr, 0, 64);
      for (int d = 0; d < 128; ++d) {
        int64_t at = mx_code_byte(is_v, p, h, H, o, d);
        int code = (code_plane[at] >> (4 * (d & 1))) & 15;
        cr[d / 2] |= (uint8_t)(code << (4 * (d & 1)));
      }
      for (int b = 0; b < 4; ++b) scales[(t * H + h) * 4 + b] = scale_plane[mx_scale_byte(is_v, p, h, H, o, b)];
    }
  }
}

static double mx_plane_value(const uint8_t* code_plane, const uint8_t* scale_plane, int is_v, int64_t s, int h, int H,
                             int d, double g) {
  (void)g;
  int64_t p = s / 16;
  int o = (int)(s % 16);
  int64_t at = mx_code_byte(is_v, p, h, H, o, d);
  int code = (code_plane[at] >> (4 * (d & 1))) & 15;
  return nvfp4o_e2m1_value(code) * nvfp4o_e8m0_value(scale_plane[mx_scale_byte(is_v, p, h, H, o, d / 32)]);
}

/* Decode attention over MXFP4 pages: the same attention as
 * nvfp4o_decode_attention with K_hat / V_hat the MXFP4 values. */
void nvfp4o_mx_decode_attention(const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int Hkv,
                                const float* q, int Hq, const int32_t* block_table, int bt_stride,
                                const int32_t* seq_lens, float sm_scale, const int64_t* rows, int64_t n_rows,
                                double* out) {
  decode_attention_with(mx_plane_value, kc, ks, vc, vs, Hkv, 1.0f, 1.0f, q, Hq, block_table, bt_stride, seq_lens,
                        sm_scale, rows, n_rows, out);
}

/* ------------------------------------------------------- Hadamard rotation
 * [TC] "E2M1 encoding and two-level scaling" section, quantization tricks: an
 * orthogonal Hadamard transform applied before quantization spreads a local
 * outlier over the whole vector.  Reading R10: K rows (128 values along
 * head_dim) are multiplied by the 128-point Sylvester Walsh-Hadamard matrix
 * H[i][j] = (-1)^popcount(i & j) times 2^-4 before NVFP4 quantization, and
 * queries by H times 2^-3 before attention: H H^T = 128 I, so the scores are
 * unchanged, q'.k' = 2^-7 q^T H^T H k = q.k, and both scales are powers of two.
 * out[r][i] = scale * sum_j H[i][j] x[r][j], summed in float64 in j order (the
 * matrix definition; exact whenever the sum fits 53 bits). */
void nvfp4o_hadamard_rows(const double* x, int64_t n_rows, double scale, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const double* xr = x + r * 128;
    for (int i = 0; i < 128; ++i) {
      double acc = 0.0;
      for (int j = 0; j < 128; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -xr[j] : xr[j];
      out[r * 128 + i] = scale * acc;
    }
  }
}

/* ------------------------------------------------- Sparse-MLA latent cache
 * [MW] §6 closing note: the serving engine's NVFP4 KV cache supports GQA and
 * Sparse MLA models.  The pages say nothing more; the readings (also in the
 * design notes):
 *   M1 an MLA cache holds one latent row per token, shared by every query
 *      head: 512 latent values followed by 64 rotary-key values (the
 *      DeepSeek-V3-class shape).  Scores use all 576 values; the output is the
 *      softmax-weighted sum of the first 512 (decode with the key and value
 *      up-projections absorbed into the query and the output projection).
 *   M2 the row is stored as NVFP4 with the GQA cache's rule: 36 blocks of 16
 *      consecutive values, E4M3 scale per block, one FP32 global scale g per
 *      layer (readings R1..R8 apply block by block).
 *   M3 "sparse": each query token attends only to a given list of cached
 *      tokens (its top-k selection, made outside this path).  List entries
 *      are cache slots; an entry outside [0, num_slots) is skipped; an entry
 *      listed twice counts twice.
 *   M4 layout: codes [num_slots][288] (byte j = values 2j, 2j+1, low nibble
 *      first), scales [num_slots][36] (byte b = E4M3 scale of values
 *      16b..16b+15); a slot is page * page_size + offset for any page size. */

#define MLA_D 576
#define MLA_DV 512

/* Latent rows [n_rows][576] -> codes [n_rows][288], scales [n_rows][36] (M2, M4). */
void nvfp4o_mla_quantize_rows(const float* x, int64_t n_rows, float g, uint8_t* codes, uint8_t* scales) {
  const double gd = (double)g;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    memset(codes + r * (MLA_D / 2), 0, MLA_D / 2);
    for (int b = 0; b < MLA_D / 16; ++b)
      quantize_block16(x + r * MLA_D + 16 * b, gd, codes + r * (MLA_D / 2) + 8 * b, scales + r * (MLA_D / 16) + b);
  }
}

/* Value d of the latent row in slot s: E2M1 * E4M3 * g, exact in float64. */
static double mla_value(const uint8_t* pc, const uint8_t* ps, int64_t s, int d, double g) {
  int code = (pc[s * (MLA_D / 2) + d / 2] >> (4 * (d & 1))) & 15;
  return nvfp4o_e2m1_value(code) * nvfp4o_e4m3_value(ps[s * (MLA_D / 16) + d / 16]) * g;
}

/* Sparse MLA decode (M1, M3): for query token t < T and head h < Hq, with the
 * valid entries j of indices[t][0..topk):
 *   s_j = sm_scale * sum_{d<576} q[t][h][d] * K_hat[slot_j][d]
 *   out[t][h][d] = sum_j softmax(s)_j * K_hat[slot_j][d],  d < 512
 * in float64; no valid entry gives zeros.  q: [T][Hq][576], out: [T][Hq][512]. */
void nvfp4o_mla_sparse_decode(const uint8_t* pc, const uint8_t* ps, int64_t num_slots, float g, const float* q,
                              int64_t T, int Hq, const int32_t* indices, int topk, float sm_scale, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t th = 0; th < T * Hq; ++th) {
    const int64_t t = th / Hq;
    const float* qr = q + th * MLA_D;
    double* o = out + th * MLA_DV;
    for (int d = 0; d < MLA_DV; ++d) o[d] = 0.0;
    double* sc = (double*)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(double));
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < topk; ++j) {
      const int64_t s = indices[t * topk + j];
      if (s < 0 || s >= num_slots) continue;
      double acc = 0.0;
      for (int d = 0; d < MLA_D; ++d) acc += (double)qr[d] * mla_value(pc, ps, s, d, (double)g);
      sc[j] = (double)sm_scale * acc;
      if (sc[j] > m) m = sc[j];
      any = 1;
    }
    if (any) {
      double l = 0.0;
      for (int j = 0; j < topk; ++j) {
        const int64_t s = indices[t * topk + j];
        if (s < 0 || s >= num_slots) continue;
        const double w = exp(sc[j] - m);
        l += w;
        for (int d = 0; d < MLA_DV; ++d) o[d] += w * mla_value(pc, ps, s, d, (double)g);
      }
      for (int d = 0; d < MLA_DV; ++d) o[d] /= l;
    }
    free(sc);
  }
}

/* ------------------------------------------- unrounded two-level scaling
 * [MW] §2 compares two-level scaling against a single global scale on
 * Gaussian data with a few large outliers; its comparison keeps the block
 * scale unrounded and has no tensor scale.  This is that rule, written with
 * the oracle's own encoder: per block of `block` values, s = amax/6 (a block
 * of zeros stays zero) and each value v becomes sign(v) * E2M1(c) * s with
 * c = nvfp4o_e2m1_encode(|v|/s) (nearest magnitude, ties to the even code --
 * ties have measure zero on such data).  block = n is the global-only
 * comparator. */
void nvfp4o_unrounded_block_dequant(const double* x, int64_t n, int64_t block, double* out) {
  for (int64_t s0 = 0; s0 < n; s0 += block) {
    const int64_t s1 = s0 + block < n ? s0 + block : n;
    double amax = 0.0;
    for (int64_t i = s0; i < s1; ++i) amax = fmax(amax, fabs(x[i]));
    const double s = amax / 6.0;
    for (int64_t i = s0; i < s1; ++i) {
      const double mag = s > 0.0 ? nvfp4o_e2m1_value(nvfp4o_e2m1_encode(fabs(x[i]) / s)) * s : 0.0;
      out[i] = copysign(mag, x[i]);
    }
  }
}

/* Bytes the cache planes take per (token, kv head): 64 code bytes + 8 scale
 * bytes for each of K and V ([MW] §1: 16 E2M1 values in 8 bytes plus one
 * E4M3 byte = 9/16 byte per value). */
int64_t nvfp4o_bytes_per_token_head(void) { return 2 * (64 + 8); }

/* Threads OpenMP will use (for the reported CPU-baseline core count). */
int nvfp4o_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
