// Plain C++ statement of the CPU oracle's MXFP8 arithmetic -- test infrastructure only.
//
// It computes, with plain loops in double precision, the same values as the NumPy oracle
// (oracle/mx.py, oracle/attention.py) for MXFP8 (E4M3) operands: the E4M3 and E8M0 codecs, the
// ROW32 / COL32 / SQ32 block quantizers, and the attention forward and backward of one (batch,
// head).  It shares no code with the HIP library and is loaded only by the tests (through
// ctypes), which check it against the NumPy oracle and against the pages' own figures.
//
// What it follows, from the pages:
//  * "Low-Precision FlashAttention-4 ... for NVIDIA Blackwell", section "Understanding OCP MXFP8
//    Microscaling on Blackwell": 32 contiguous elements share one E8M0 scale 2^(code - 127), each
//    element an 8-bit FP8 (E4M3) value.
//  * same page, section "1. End-to-End Block-Scaled GEMM Fusion": S = Q K^T and P V are products
//    of MX operands; section "2. Synchronized Online Softmax with Dynamic Scaling": the softmax in
//    fp32 with the logits scaled by softmax_scale.
//  * "Low Precision Flash Attention 4: End-to-End Block-Scaled Attention for Blackwell", the
//    forward/backward paragraph: P goes to MXFP8 before P V with scales from the row maximum; the
//    backward quantizes Q, K and dO in square [32, 32] blocks, recomputes P and quantizes dS online
//    in square blocks (contributions paragraph).
// Where the pages are silent it takes the readings the NumPy oracle states (E4M3 "FN", round to
// nearest even with saturation at 448; scale code floor(log2 amax) - 8 + 127 clamped to [0, 254];
// a log2-domain softmax with c = fl32(fl32(sigma) fl32(log2 e)) and an integer row frame
// M = ceil(fl32(max S c)); the normalizer l summing the unquantized p; P-hat in blocks of 32 keys
// per query for P V and of 32 queries per key for dV = P^T dO; every product of MX operands the
// exact sum rounded once to fp32).  fl32() marks one rounding to float32; every other sum is double.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

namespace {

constexpr int kBlock = 32;

double fl32(double x) { return static_cast<double>(static_cast<float>(x)); }

// E4M3 "FN": sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities, S.1111.111 is NaN,
// exponent field 0 holds the subnormals m 2^-9.
double e4m3_value(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 0)
    mag = std::ldexp(static_cast<double>(m), -9);
  else if (e == 15 && m == 7)
    mag = NAN;
  else
    mag = std::ldexp(static_cast<double>(8 + m), e - 10);
  return (code & 0x80) ? -mag : mag;
}

// Round to the nearest E4M3 value, ties to even mantissa, saturating at +-448 (code 0x7E);
// the sign bit is kept (so -0 is 0x80).  nearbyint rounds ties to even in the default mode.
uint8_t e4m3_code(double y) {
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  const double a = std::fabs(y);
  if (std::isnan(a)) return sign | 0x7F;   // outside the quantizer's contract; the format's NaN code
  if (std::isinf(a)) return sign | 0x7E;
  if (a < std::ldexp(1.0, -6)) {   // subnormal binade: multiples of 2^-9 (8 x 2^-9 is the smallest normal)
    return sign | static_cast<uint8_t>(std::nearbyint(a * 512.0));
  }
  int ex;
  std::frexp(a, &ex);   // a = f 2^ex, f in [0.5, 1)
  int e = ex - 1;       // floor(log2 a)
  int m = static_cast<int>(std::nearbyint((std::ldexp(a, -e) - 1.0) * 8.0));
  if (m == 8) {         // the mantissa rounded up into the next binade
    m = 0;
    ++e;
  }
  if (e > 8 || (e == 8 && m == 7)) return sign | 0x7E;
  return sign | static_cast<uint8_t>(((e + 7) << 3) | m);
}

// E8M0 code of a block from its largest magnitude: floor(log2 amax) - 8 + 127 (8 = the exponent of
// E4M3's largest power of two), clamped to [0, 254]; an all-zero block takes code 0.
uint8_t scale_code(double amax) {
  if (amax == 0.0) return 0;
  int ex;
  std::frexp(amax, &ex);
  int k = (ex - 1) - 8 + 127;
  if (k < 0) k = 0;
  if (k > 254) k = 254;
  return static_cast<uint8_t>(k);
}

double e8m0_value(uint8_t k) { return std::ldexp(1.0, static_cast<int>(k) - 127); }

// Quantize one block given as n values at x[0], x[stride], ...: codes at the same positions of c.
uint8_t quantize_block(const double* x, long stride, int n, uint8_t* c) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::fmax(amax, std::fabs(x[i * stride]));
  const uint8_t k = scale_code(amax);
  for (int i = 0; i < n; ++i) c[i * stride] = e4m3_code(std::ldexp(x[i * stride], 127 - static_cast<int>(k)));
  return k;
}

// Row-major x [n, d]: blocks of 32 along each row; scales [n, d/32] (d a multiple of 32).
void quantize_row32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  for (int r = 0; r < n; ++r)
    for (int b = 0; b < d / kBlock; ++b)
      scales[(long)r * (d / kBlock) + b] =
          quantize_block(x + (long)r * d + kBlock * b, 1, kBlock, codes + (long)r * d + kBlock * b);
}

// Blocks of 32 consecutive rows in each column (aligned at row 0, a short tail block holding the
// rest); scales [ceil(n/32), d].
void quantize_col32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  for (int rb = 0; rb * kBlock < n; ++rb) {
    const int rows = std::min(kBlock, n - rb * kBlock);
    for (int col = 0; col < d; ++col)
      scales[(long)rb * d + col] =
          quantize_block(x + (long)rb * kBlock * d + col, d, rows, codes + (long)rb * kBlock * d + col);
  }
}

// Square blocks of 32 rows x 32 columns aligned at (0, 0), short tail blocks along either axis;
// scales [ceil(n/32), ceil(d/32)].
void quantize_sq32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  const int nbc = (d + kBlock - 1) / kBlock;
  for (int rb = 0; rb * kBlock < n; ++rb)
    for (int cb = 0; cb < nbc; ++cb) {
      const int r0 = rb * kBlock, c0 = cb * kBlock;
      const int rows = std::min(kBlock, n - r0), cols = std::min(kBlock, d - c0);
      double amax = 0.0;
      for (int r = r0; r < r0 + rows; ++r)
        for (int c = c0; c < c0 + cols; ++c) amax = std::fmax(amax, std::fabs(x[(long)r * d + c]));
      const uint8_t k = scale_code(amax);
      scales[(long)rb * nbc + cb] = k;
      for (int r = r0; r < r0 + rows; ++r)
        for (int c = c0; c < c0 + cols; ++c)
          codes[(long)r * d + c] = e4m3_code(std::ldexp(x[(long)r * d + c], 127 - static_cast<int>(k)));
    }
}

// Dequantized values of the three layouts (row-major [n, d]).
std::vector<double> values_row32(const double* x, int n, int d) {
  std::vector<uint8_t> c((size_t)n * d), s((size_t)n * (d / kBlock));
  quantize_row32(x, n, d, c.data(), s.data());
  std::vector<double> v((size_t)n * d);
  for (int r = 0; r < n; ++r)
    for (int j = 0; j < d; ++j)
      v[(size_t)r * d + j] = e4m3_value(c[(size_t)r * d + j]) * e8m0_value(s[(size_t)r * (d / kBlock) + j / kBlock]);
  return v;
}

std::vector<double> values_col32(const double* x, int n, int d) {
  std::vector<uint8_t> c((size_t)n * d), s((size_t)((n + kBlock - 1) / kBlock) * d);
  quantize_col32(x, n, d, c.data(), s.data());
  std::vector<double> v((size_t)n * d);
  for (int r = 0; r < n; ++r)
    for (int j = 0; j < d; ++j) v[(size_t)r * d + j] = e4m3_value(c[(size_t)r * d + j]) * e8m0_value(s[(size_t)(r / kBlock) * d + j]);
  return v;
}

std::vector<double> values_sq32(const double* x, int n, int d) {
  const int nbc = (d + kBlock - 1) / kBlock;
  std::vector<uint8_t> c((size_t)n * d), s((size_t)((n + kBlock - 1) / kBlock) * nbc);
  quantize_sq32(x, n, d, c.data(), s.data());
  std::vector<double> v((size_t)n * d);
  for (int r = 0; r < n; ++r)
    for (int j = 0; j < d; ++j)
      v[(size_t)r * d + j] = e4m3_value(c[(size_t)r * d + j]) * e8m0_value(s[(size_t)(r / kBlock) * nbc + j / kBlock]);
  return v;
}

// c = fl32(fl32(sigma) fl32(log2 e))
const double kLog2e32 = fl32(1.4426950408889634);
double log2_scale(double sigma) { return fl32(fl32(sigma) * kLog2e32); }

bool visible(int i, int j, bool causal) { return !causal || j <= i; }

}  // namespace

extern "C" {

double mxo_e4m3_value(uint8_t code) { return e4m3_value(code); }
uint8_t mxo_e4m3_code(double y) { return e4m3_code(y); }
uint8_t mxo_scale_code(double amax) { return scale_code(amax); }

void mxo_quantize_row32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  quantize_row32(x, n, d, codes, scales);
}
void mxo_quantize_col32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  quantize_col32(x, n, d, codes, scales);
}
void mxo_quantize_sq32(const double* x, int n, int d, uint8_t* codes, uint8_t* scales) {
  quantize_sq32(x, n, d, codes, scales);
}

// Forward of one head: q, k, v [L, d] source values (row-major doubles).  Writes O [L, d] (before
// any output cast), LSE [L] (natural log), and, when the pointers are non-null, the P-hat codes
// [L, L] (0 where masked) and scales [L, ceil(L/32)] (blocks of 32 keys per query).
void mxo_attn_fwd(const double* q, const double* k, const double* v, int L, int d, double sigma, int causal,
                  double* O, double* LSE, uint8_t* p_codes, uint8_t* p_scales) {
  const std::vector<double> qh = values_row32(q, L, d), kh = values_row32(k, L, d), vh = values_col32(v, L, d);
  const double c = log2_scale(sigma);
  const int nkb = (L + kBlock - 1) / kBlock;
  std::vector<double> S((size_t)L), p((size_t)L), ph((size_t)L);
  std::vector<uint8_t> pc((size_t)L);
  for (int i = 0; i < L; ++i) {
    double smax = -INFINITY;
    for (int j = 0; j < L; ++j) {
      double acc = 0.0;
      for (int t = 0; t < d; ++t) acc += qh[(size_t)i * d + t] * kh[(size_t)j * d + t];
      S[j] = fl32(acc);
      if (visible(i, j, causal)) smax = std::fmax(smax, S[j]);
    }
    const double M = std::ceil(fl32(smax * c));
    double l = 0.0;
    for (int j = 0; j < L; ++j) {
      p[j] = visible(i, j, causal) ? fl32(std::exp2(fl32(S[j] * c - M))) : 0.0;
      l += p[j];
    }
    // P-hat: blocks of 32 keys of this query
    for (int b = 0; b < nkb; ++b) {
      const int n = std::min(kBlock, L - kBlock * b);
      const uint8_t kb = quantize_block(p.data() + kBlock * b, 1, n, pc.data() + kBlock * b);
      if (p_scales) p_scales[(size_t)i * nkb + b] = kb;
      for (int j = kBlock * b; j < kBlock * b + n; ++j) ph[j] = e4m3_value(pc[j]) * e8m0_value(kb);
    }
    if (p_codes)
      for (int j = 0; j < L; ++j) p_codes[(size_t)i * L + j] = pc[j];
    for (int t = 0; t < d; ++t) {
      double acc = 0.0;
      for (int j = 0; j < L; ++j) acc += ph[j] * vh[(size_t)j * d + t];
      O[(size_t)i * d + t] = acc / l;
    }
    LSE[i] = std::log(2.0) * (M + std::log2(l));
  }
}

// Backward of one head: q, k, v, o, dout [L, d], lse [L] (the forward's fp32 values).  Writes
// dQ, dK, dV [L, d] (double, before any output cast) and D [L].
void mxo_attn_bwd(const double* q, const double* k, const double* v, const double* o, const double* dout,
                  const double* lse, int L, int d, double sigma, int causal, double* dQ, double* dK, double* dV,
                  double* Dv) {
  const std::vector<double> qs = values_sq32(q, L, d), ks = values_sq32(k, L, d), dos = values_sq32(dout, L, d);
  const std::vector<double> vr = values_row32(v, L, d);
  const double c = log2_scale(sigma);
  std::vector<double> p((size_t)L * L), dS((size_t)L * L);
  for (int i = 0; i < L; ++i) {
    double acc = 0.0;
    for (int t = 0; t < d; ++t) acc += dout[(size_t)i * d + t] * o[(size_t)i * d + t];
    Dv[i] = fl32(acc);
  }
  for (int i = 0; i < L; ++i) {
    const double l2 = fl32(lse[i] * kLog2e32);
    for (int j = 0; j < L; ++j) {
      if (!visible(i, j, causal)) {
        p[(size_t)i * L + j] = dS[(size_t)i * L + j] = 0.0;
        continue;
      }
      double s = 0.0, dp = 0.0;
      for (int t = 0; t < d; ++t) {
        s += qs[(size_t)i * d + t] * ks[(size_t)j * d + t];
        dp += dos[(size_t)i * d + t] * vr[(size_t)j * d + t];
      }
      const double pij = fl32(std::exp2(fl32(fl32(s) * c - l2)));
      p[(size_t)i * L + j] = pij;
      dS[(size_t)i * L + j] = fl32(pij * fl32(fl32(dp) - Dv[i]));
    }
  }
  // dS-hat in [32 queries x 32 keys] blocks; P-hat for dV in blocks of 32 queries per key
  const std::vector<double> dSh = values_sq32(dS.data(), L, L), pb = values_col32(p.data(), L, L);
  for (int j = 0; j < L; ++j)
    for (int t = 0; t < d; ++t) {
      double av = 0.0, ak = 0.0;
      for (int i = 0; i < L; ++i) {
        av += pb[(size_t)i * L + j] * dos[(size_t)i * d + t];
        ak += dSh[(size_t)i * L + j] * qs[(size_t)i * d + t];
      }
      dV[(size_t)j * d + t] = av;
      dK[(size_t)j * d + t] = sigma * ak;
    }
  for (int i = 0; i < L; ++i)
    for (int t = 0; t < d; ++t) {
      double aq = 0.0;
      for (int j = 0; j < L; ++j) aq += dSh[(size_t)i * L + j] * ks[(size_t)j * d + t];
      dQ[(size_t)i * d + t] = sigma * aq;
    }
}

}  // extern "C"
