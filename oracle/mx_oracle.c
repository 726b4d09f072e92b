/*
 * Plain CPU oracle for the MXFP4 weight-streaming MoE layer and the dense
 * MXFP4 linear layer.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and
 * the CPU-baseline leg of the benchmark load it; the product path never does.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Sources (the pages define the format; the remaining steps are the plainest
 * reading of the layer they describe):
 *   - "Zyphra Inference Wave 2" (aihot.news mirror), section "Quantization.":
 *     MXFP4 = blocks of 32 values sharing one 8-bit power-of-two scale, each
 *     value a 4-bit float with magnitude in {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *     4.25 bits per value.
 *   - same page, "Quantization" (serving) section: an MXFP4 expert runs the two
 *     expert GEMMs and combines the results; only the routed experts are read.
 *   - same page, section "Speculative decoding.": a step of T tokens reads each
 *     needed weight once and applies it to every token of the step.
 *   - "Bringing Ultra-Fast, Interactive LLM Inference to AMD Instinct MI355X
 *     GPUs" (AMD ROCm blog), section "3. Low-Precision Data Types": 4-bit
 *     values with one shared scale per 32, fed to the matrix instructions
 *     with MXFP8 activations (the *_a8 functions below).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - E2M1 code c: sign = bit 3, bits 2..0 index the eight magnitudes in
 *     ascending order; code 8 is -0.0.
 *   - E8M0 byte s: value 2^(s-127); s = 0xFF is NaN; no zero, no infinity.
 *   - Packing: codes of a row are K-contiguous, two per byte, element 2i in the
 *     low nibble and 2i+1 in the high nibble; one scale byte per 32
 *     consecutive K values of one output row.
 *   - Weight tensors are row-major [rows = output features][K/2] bytes plus
 *     scales [rows][K/32]; the gate_up tensor holds the I gate rows first,
 *     then the I up rows.
 *   - Router: the k largest logits (ties to the lower expert id), slots in
 *     descending-logit order; gates are a softmax over the k selected logits.
 *   - SwiGLU: h = silu(g) * u, silu(g) = g / (1 + exp(-g)); h is rounded once
 *     to bf16 (round to nearest even).
 *   - Accumulation: fp32, K ascending, each product rounded to fp32 first;
 *     the combine sums the k gate-weighted fp32 down outputs in slot order and
 *     rounds once to bf16.
 *   - MXFP8 activations (the *_a8 functions): the OCP MX format with E4M3
 *     elements (bias 7, no infinities, S.1111.111 = NaN, largest 448).  Per
 *     block of 32 consecutive K values of one activation row, the E8M0 scale
 *     is 2^(floor(log2 amax) - 8) (8 = exponent of E4M3's largest value),
 *     clamped to the E8M0 range, and each value divided by it is rounded to
 *     the nearest E4M3 value (ties to even), saturating at +-448.  An all-zero
 *     block gets scale byte 0; a block holding a NaN or an infinity gets
 *     scale 0xFF (NaN) and codes 0x7F.  The MoE layer quantizes x before the
 *     gate_up GEMM and the bf16 h before the down GEMM.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * Contraction and fast-math are off so every fp32 operation is one IEEE
 * rounding and results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_VERSION 2

int ora_version(void) { return ORA_VERSION; }

/* ---------------------------------------------------------------- format */

/* E2M1 magnitudes, ascending ("Quantization." section of the Zyphra page). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double ora_e2m1(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m; /* code 8 gives -0.0 */
}

/* E8M0 scale: an 8-bit power of two with bias 127; 0xFF encodes NaN. */
double ora_e8m0(int s) {
  if ((s & 0xFF) == 0xFF) return NAN;
  return ldexp(1.0, (s & 0xFF) - 127);
}

/* Nibble i of a packed row: element 2j is the low nibble of byte j. */
static int nibble(const uint8_t* row, int64_t i) {
  uint8_t b = row[i >> 1];
  return (i & 1) ? (b >> 4) : (b & 15);
}

/* Pack n 4-bit codes (n even) into n/2 bytes, element 2j in the low nibble. */
void ora_pack_codes(const uint8_t* codes, int64_t n, uint8_t* packed) {
  for (int64_t j = 0; j < n / 2; ++j)
    packed[j] = (uint8_t)((codes[2 * j] & 15) | ((codes[2 * j + 1] & 15) << 4));
}

void ora_unpack_codes(const uint8_t* packed, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)nibble(packed, i);
}

/* Exact weight value w[r,k] = e2m1(code) * 2^(s-127), in fp64 (exact: at most
 * two significant bits, exponent within fp64 range). */
static double weight(const uint8_t* w, const uint8_t* s, int64_t K, int64_t r, int64_t k) {
  return ora_e2m1(nibble(w + r * (K / 2), k)) * ora_e8m0(s[r * (K / 32) + k / 32]);
}

/* Dequantize rows x K weights to fp64. */
void ora_dequant_f64(const uint8_t* w, const uint8_t* s, int64_t rows, int64_t K, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = weight(w, s, K, r, k);
}

/* ------------------------------------------------------------ bf16 helpers */

static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), overflow to +-Inf, NaN
 * kept.  bf16 = 1 sign, 8 exponent (bias 127), 7 stored fraction bits. */
uint16_t ora_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a == 0.0) return neg ? 0x8000 : 0x0000;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  int qexp = e - 8;          /* 8 significant bits */
  if (qexp < -133) qexp = -133; /* subnormal spacing 2^-133 */
  double q = ldexp(1.0, qexp);
  double n = nearbyint(a / q); /* exact division by a power of two; ties-to-even */
  double r = n * q;
  uint16_t bits;
  if (r > 3.3895313892515355e38) { /* largest finite bf16, (2 - 2^-7) * 2^127 */
    bits = 0x7F80;
  } else {
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    bits = (uint16_t)(u >> 16);
  }
  return (uint16_t)(bits | (neg ? 0x8000 : 0));
}

/* ---------------------------------------------------------- dense linear */

/* One fp32 dot product: acc = fl32(acc + fl32(x_k * w_k)), K ascending.
 * Also returns sum_k |x_k * w_k| in fp64 (the scale of the acceptance bound). */
static float dot_row(const uint16_t* x, const uint8_t* w, const uint8_t* s, int64_t K, int64_t r,
                     double* abs_sum) {
  float acc = 0.0f;
  double as = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double xv = bf16_to_f64(x[k]);
    double wv = weight(w, s, K, r, k);
    double p = xv * wv; /* exact in fp64 */
    float pf = (float)p;
    acc = acc + pf;
    as += fabs(p);
  }
  if (abs_sum) *abs_sum = as;
  return acc;
}

/* The same dot product over activations given as exact fp64 values. */
static float dot_vals(const double* a, const uint8_t* w, const uint8_t* s, int64_t K, int64_t r,
                      double* abs_sum) {
  float acc = 0.0f;
  double as = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = a[k] * weight(w, s, K, r, k); /* exact in fp64 */
    float pf = (float)p;
    acc = acc + pf;
    as += fabs(p);
  }
  if (abs_sum) *abs_sum = as;
  return acc;
}

/* y[t,n] = bf16(sum_k x[t,k] * w[n,k]).  x: bf16 bits [T,K]; w: [N,K/2];
 * s: [N,K/32].  Outputs: y bf16 bits [T,N]; acc fp32 [T,N] (may be NULL);
 * scale_d fp64 [T,N] = sum_k |x*w| (may be NULL). */
void ora_mx_linear(const uint16_t* x, const uint8_t* w, const uint8_t* s, int64_t T, int64_t K,
                   int64_t N, uint16_t* y, float* acc, double* scale_d, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) collapse(2)
#endif
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      double as;
      float a = dot_row(x + t * K, w, s, K, n, &as);
      if (y) y[t * N + n] = ora_bf16_rne((double)a);
      if (acc) acc[t * N + n] = a;
      if (scale_d) scale_d[t * N + n] = as;
    }
}

/* ----------------------------------------------------- MXFP8 activations */

/* E4M3 code -> value: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
 * 2..0; exponent field 0 holds subnormals m * 2^-9; 0x7F / 0xFF are NaN. */
double ora_e4m3(int code) {
  code &= 0xFF;
  int sg = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return sg ? -v : v;
}

/* Magnitude code (bits 6..0) of the E4M3 value nearest to a >= 0 (finite),
 * ties to the even mantissa, saturating at 448. */
static int e4m3_magnitude(double a) {
  if (a >= 448.0) return 0x7E;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): leading bit 2^(e-1) */
  int lead = e - 1;
  if (a == 0.0 || lead < -6) lead = -6; /* below 2^-6 the spacing is 2^-9 */
  double q = ldexp(1.0, lead - 3);      /* 3 fraction bits */
  double r = nearbyint(a / q) * q;      /* exact division; ties to even */
  if (r < ldexp(1.0, -6)) return (int)(r / ldexp(1.0, -9)); /* subnormal */
  int er;
  double fr = frexp(r, &er); /* r < 448 before rounding, so r <= 448 here */
  int ex = er - 1 + 7;
  int m = (int)((fr * 2.0 - 1.0) * 8.0);
  return (ex << 3) | m;
}

/* Quantize rows x K bf16 activations (K % 32 == 0) to MXFP8: codes [rows,K]
 * (one E4M3 byte per value), scales [rows,K/32] (E8M0 bytes). */
void ora_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 32; ++b) {
      const uint16_t* blk = x + r * K + 32 * b;
      uint8_t* cb = codes + r * K + 32 * b;
      double amax = 0.0;
      int finite = 1;
      for (int i = 0; i < 32; ++i) {
        double v = bf16_to_f64(blk[i]);
        if (!isfinite(v)) finite = 0;
        else if (fabs(v) > amax) amax = fabs(v);
      }
      if (!finite) {
        scales[r * (K / 32) + b] = 0xFF;
        for (int i = 0; i < 32; ++i) cb[i] = 0x7F;
        continue;
      }
      int sbyte = 0;
      if (amax > 0.0) {
        int e;
        frexp(amax, &e);
        sbyte = (e - 1) - 8 + 127;
        if (sbyte < 0) sbyte = 0;
        if (sbyte > 254) sbyte = 254;
      }
      scales[r * (K / 32) + b] = (uint8_t)sbyte;
      double scale = ldexp(1.0, sbyte - 127);
      for (int i = 0; i < 32; ++i) {
        double v = bf16_to_f64(blk[i]) / scale; /* exact: a power of two */
        cb[i] = (uint8_t)((signbit(v) ? 0x80 : 0) | e4m3_magnitude(fabs(v)));
      }
    }
}

/* One activation row as the GEMM sees it: exact fp64 values of the row
 * (bf16 as is, or quantized to MXFP8 and decoded when act8 is set). */
static void activation_row(const uint16_t* x, int64_t K, int act8, double* out) {
  if (!act8) {
    for (int64_t k = 0; k < K; ++k) out[k] = bf16_to_f64(x[k]);
    return;
  }
  uint8_t* c = (uint8_t*)malloc((size_t)K);
  uint8_t* s = (uint8_t*)malloc((size_t)(K / 32));
  ora_mxfp8_quantize(x, 1, K, c, s);
  for (int64_t k = 0; k < K; ++k) out[k] = ora_e4m3(c[k]) * ora_e8m0(s[k / 32]);
  free(c);
  free(s);
}

/* The dense layer with MXFP8 activations: y[t,n] = bf16(sum_k q(x)[t,k] w[n,k]),
 * q(x) the MXFP8-quantized x (K % 32 == 0).  Outputs as ora_mx_linear;
 * scale_d = sum_k |q(x) * w|. */
void ora_mx_linear_a8(const uint16_t* x, const uint8_t* w, const uint8_t* s, int64_t T, int64_t K,
                      int64_t N, uint16_t* y, float* acc, double* scale_d, int nthreads) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(T * K));
  for (int64_t t = 0; t < T; ++t) activation_row(x + t * K, K, 1, a + t * K);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) collapse(2)
#endif
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      double as;
      float v = dot_vals(a + t * K, w, s, K, n, &as);
      if (y) y[t * N + n] = ora_bf16_rne((double)v);
      if (acc) acc[t * N + n] = v;
      if (scale_d) scale_d[t * N + n] = as;
    }
  free(a);
}

/* ---------------------------------------------------------------- routing */

/* For each token: the k largest logits, ties to the lower expert id, slots in
 * descending-logit order; gate_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * evaluated in fp64 and stored as fp32.  Logits must be finite. */
void ora_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids, float* gates) {
  char* taken = (char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      taken[best] = 1;
      ids[t * k + j] = (int32_t)best;
    }
    double m = (double)l[ids[t * k]];
    double den = 0.0;
    for (int64_t j = 0; j < k; ++j) den += exp((double)l[ids[t * k + j]] - m);
    for (int64_t j = 0; j < k; ++j) gates[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - m) / den);
  }
  free(taken);
}

/* ------------------------------------------------------------ expert sort */

/* Counting sort of the T*k flat slots f = t*k + j by expert id: experts
 * ascending, f ascending within an expert (a stable sort by expert).  The
 * pages say only that a step's tokens are grouped by the expert they route to
 * so that each routed expert's weights are read once ("Zyphra Inference Wave
 * 2", sections "Speculative decoding." and "Quantization"); the stable order
 * is the plainest reading.  Outputs: counts [E]; offsets [E+1] (exclusive
 * prefix sums); sorted_slots [T*k]; active [E] = the experts with at least one
 * slot, ascending (entries past the count are set to -1); *num_active = their
 * number.  The order in which a GPU takes the active experts is its own
 * scheduling choice and is not part of this definition. */
void ora_sort(const int32_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts, int32_t* offsets,
              int32_t* sorted_slots, int32_t* active, int32_t* num_active) {
  if (E < 1) return;
  int64_t F = T * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < F; ++f) counts[ids[f]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t f = 0; f < F; ++f) {
    int32_t e = ids[f];
    sorted_slots[offsets[e] + fill[e]] = (int32_t)f;
    fill[e] += 1;
  }
  free(fill);
  int32_t na = 0;
  for (int64_t e = 0; e < E; ++e)
    if (counts[e] > 0) active[na++] = (int32_t)e;
  for (int64_t e = na; e < E; ++e) active[e] = -1;
  *num_active = na;
}

/* ------------------------------------------------------------- MoE layer */

/* silu(g) * u in fp64 from the fp32 g and u. */
static double swiglu(float g, float u) {
  double gd = (double)g;
  return gd / (1.0 + exp(-gd)) * (double)u;
}

/* MoE forward for the tokens listed in tok[0..ntok): each token routes to its
 * k routed slots (ora_route over the E logits) and then to the n_shared shared
 * experts E .. E + n_shared - 1 with gate 1 (a model's always-active experts);
 * for each token t and slot j < k + n_shared (expert e = ids[t,j], gate = gates[t,j]):
 *   g_n = sum_K x[t,K] Wgu[e][n,K],  u_n = sum_K x[t,K] Wgu[e][I+n,K]   (fp32)
 *   h_n = bf16(silu(g_n) * u_n)                                         n < I
 *   d_n = sum_i h_i Wd[e][n,i]                                          (fp32)
 *   y[t,n] = bf16(sum_j fl32(gate_j * d_{j,n}))  j ascending, fp32.
 * Shapes: x bf16 [T,H]; logits f32 [T,E]; Wgu [E+n_shared,2I,H/2],
 * Sgu [E+n_shared,2I,H/32]; Wd [E+n_shared,H,I/2], Sd [E+n_shared,H,I/32].
 * Outputs indexed by position in tok: y [ntok,H] bf16 bits;
 * scale_m [ntok,H] = sum_j gate_j sum_i |h_i Wd[e][n,i]| (fp64, may be NULL);
 * h [ntok*(k+n_shared), I] bf16 bits (may be NULL).
 * With act8 set, x (before gate_up) and h (before down) are MXFP8-quantized
 * per block of 32 (ora_mxfp8_quantize) and the GEMMs read the quantized
 * values; h_out still returns the bf16 h and scale_m uses the quantized h. */
static void moe_tokens_impl(const uint16_t* x, const float* logits, int64_t k_routed, int64_t n_shared,
                            const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd, const uint8_t* sd,
                            int64_t H, int64_t I, int64_t E, const int32_t* tok, int64_t ntok, uint16_t* y,
                            double* scale_m, uint16_t* h_out, float* g_out, float* u_out, double* gabs_out,
                            double* uabs_out, int nthreads, int act8) {
  const int64_t k = k_routed + n_shared;  /* slots per token */
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ntok * k));
  float* gates = (float*)malloc(sizeof(float) * (size_t)(ntok * k));
  for (int64_t i = 0; i < ntok; ++i) {
    ora_route(logits + (int64_t)tok[i] * E, 1, E, k_routed, ids + i * k, gates + i * k);
    for (int64_t s = 0; s < n_shared; ++s) {
      ids[i * k + k_routed + s] = (int32_t)(E + s);
      gates[i * k + k_routed + s] = 1.0f;
    }
  }

  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(ntok * k * I));
  double* xa = (double*)malloc(sizeof(double) * (size_t)(ntok * H)); /* gate_up activations */
  double* ha = (double*)malloc(sizeof(double) * (size_t)(ntok * k * I)); /* down activations */
  for (int64_t i = 0; i < ntok; ++i) activation_row(x + (int64_t)tok[i] * H, H, act8, xa + i * H);
  const int64_t gu_rows = 2 * I;
  const size_t gu_w = (size_t)gu_rows * (size_t)(H / 2), gu_s = (size_t)gu_rows * (size_t)(H / 32);
  const size_t d_w = (size_t)H * (size_t)(I / 2), d_s = (size_t)H * (size_t)(I / 32);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) collapse(2)
#endif
  for (int64_t p = 0; p < ntok * k; ++p)
    for (int64_t n = 0; n < I; ++n) {
      int64_t e = ids[p];
      const uint8_t* W = wgu + (size_t)e * gu_w;
      const uint8_t* S = sgu + (size_t)e * gu_s;
      double ga, ua;
      float g = dot_vals(xa + (p / k) * H, W, S, H, n, &ga);
      float u = dot_vals(xa + (p / k) * H, W, S, H, I + n, &ua);
      h[p * I + n] = ora_bf16_rne(swiglu(g, u));
      if (g_out) g_out[p * I + n] = g;
      if (u_out) u_out[p * I + n] = u;
      if (gabs_out) gabs_out[p * I + n] = ga;
      if (uabs_out) uabs_out[p * I + n] = ua;
    }
  for (int64_t p = 0; p < ntok * k; ++p) activation_row(h + p * I, I, act8, ha + p * I);
#ifdef _OPENMP
#pragma omp parallel for schedule(static) collapse(2)
#endif
  for (int64_t i = 0; i < ntok; ++i)
    for (int64_t n = 0; n < H; ++n) {
      float acc = 0.0f;
      double sm = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        int64_t p = i * k + j;
        int64_t e = ids[p];
        double as;
        float d = dot_vals(ha + p * I, wd + (size_t)e * d_w, sd + (size_t)e * d_s, I, n, &as);
        float gd = (float)((double)gates[p] * (double)d);
        acc = acc + gd;
        sm += (double)gates[p] * as;
      }
      y[i * H + n] = ora_bf16_rne((double)acc);
      if (scale_m) scale_m[i * H + n] = sm;
    }
  if (h_out) memcpy(h_out, h, sizeof(uint16_t) * (size_t)(ntok * k * I));
  free(ha);
  free(xa);
  free(h);
  free(gates);
  free(ids);
}

void ora_moe_tokens(const uint16_t* x, const float* logits, int64_t k_routed, int64_t n_shared,
                    const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd, const uint8_t* sd, int64_t T,
                    int64_t H, int64_t I, int64_t E, const int32_t* tok, int64_t ntok, uint16_t* y,
                    double* scale_m, uint16_t* h_out, int nthreads) {
  (void)T;
  moe_tokens_impl(x, logits, k_routed, n_shared, wgu, sgu, wd, sd, H, I, E, tok, ntok, y, scale_m, h_out, NULL,
                  NULL, NULL, NULL, nthreads, 0);
}

/* The MoE layer with MXFP8 activations (see moe_tokens_impl). */
void ora_moe_tokens_a8(const uint16_t* x, const float* logits, int64_t k_routed, int64_t n_shared,
                       const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd, const uint8_t* sd, int64_t T,
                       int64_t H, int64_t I, int64_t E, const int32_t* tok, int64_t ntok, uint16_t* y,
                       double* scale_m, uint16_t* h_out, int nthreads) {
  (void)T;
  moe_tokens_impl(x, logits, k_routed, n_shared, wgu, sgu, wd, sd, H, I, E, tok, ntok, y, scale_m, h_out, NULL,
                  NULL, NULL, NULL, nthreads, 1);
}

/* The MoE layer (bf16 activations) with the gate_up terms of every slot row p
 * (token tok[p / (k_routed + n_shared)], slot p % (k_routed + n_shared)) and
 * column n < I: g_out, u_out = the fp32 g and u before SwiGLU, gabs_out,
 * uabs_out = sum_K |x w| of the gate and up rows in fp64 (each [ntok*k, I],
 * any may be NULL).  Other arguments and outputs as ora_moe_tokens. */
void ora_moe_tokens_terms(const uint16_t* x, const float* logits, int64_t k_routed, int64_t n_shared,
                          const uint8_t* wgu, const uint8_t* sgu, const uint8_t* wd, const uint8_t* sd, int64_t T,
                          int64_t H, int64_t I, int64_t E, const int32_t* tok, int64_t ntok, uint16_t* y,
                          double* scale_m, uint16_t* h_out, float* g_out, float* u_out, double* gabs_out,
                          double* uabs_out, int nthreads) {
  (void)T;
  moe_tokens_impl(x, logits, k_routed, n_shared, wgu, sgu, wd, sd, H, I, E, tok, ntok, y, scale_m, h_out, g_out,
                  u_out, gabs_out, uabs_out, nthreads, 0);
}
