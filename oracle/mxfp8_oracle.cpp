/*
 * mxfp8_oracle.cpp -- TEST INFRASTRUCTURE ONLY (see mxfp8_oracle.h).
 *
 * Plain loops in fp64.  Each function states the passage of the pages it
 * follows; where the pages leave a step open, the comment names the reading
 * taken.  Built with -ffp-contract=off so that every fp32 rounding written
 * here happens exactly where it is written.
 */
#include "mxfp8_oracle.h"

#include <algorithm>
#define _USE_MATH_DEFINES
#include <cmath>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

/* ------------------------------------------------------------------------- */
/* Element formats.  The pages name MXFP8 and float8_e5m2 without fixing the
 * variant; the reading taken is the OCP MX element formats:
 *   E4M3 (E4M3FN): bias 7, no infinities, S.1111.111 is NaN, max 448.
 *   E5M2:          bias 15, IEEE-like, max finite 57344.                     */
struct Fmt {
  int mbits;          /* stored mantissa bits                      */
  int bias;           /* exponent bias                             */
  int emax;           /* floor(log2(largest finite value))         */
  double maxval;      /* largest finite magnitude                  */
  double min_normal;  /* smallest normal magnitude                 */
  double sub_step;    /* spacing of the subnormal grid             */
  int maxcode;        /* code of +maxval                           */
};
const Fmt kE4M3 = {3, 7, 8, 448.0, 0x1p-6, 0x1p-9, 0x7E};
const Fmt kE5M2 = {2, 15, 15, 57344.0, 0x1p-14, 0x1p-16, 0x7B};

const Fmt* fmt_of(int fmt) { return fmt == 0 ? &kE4M3 : (fmt == 1 ? &kE5M2 : nullptr); }

double decode(int code, const Fmt& f) {
  const int s = (code >> 7) & 1;
  const int ebits = 7 - f.mbits;
  const int e = (code >> f.mbits) & ((1 << ebits) - 1);
  const int m = code & ((1 << f.mbits) - 1);
  if (f.mbits == 3 && e == 15 && m == 7) return NAN;
  if (f.mbits == 2 && e == 31) return m == 0 ? (s ? -INFINITY : INFINITY) : NAN;
  double v = (e == 0) ? m * f.sub_step : std::ldexp(1.0 + m / double(1 << f.mbits), e - f.bias);
  return s ? -v : v;
}

/* Round y (finite) to the element grid: nearest value, ties to the even
 * code, magnitudes at or above the largest finite value saturate to it, and
 * the sign bit is always kept (so -0 encodes as 0x80). */
int encode(double y, const Fmt& f) {
  const int s = std::signbit(y) ? 0x80 : 0;
  const double a = std::fabs(y);
  if (a >= f.maxval) return s | f.maxcode;
  if (a < f.min_normal) return s | int(std::nearbyint(a / f.sub_step));
  int ex;
  std::frexp(a, &ex);
  int e = ex - 1;                                   /* a in [2^e, 2^(e+1)) */
  const double frac = std::ldexp(a, -e) - 1.0;      /* exact, in [0,1)     */
  int q = int(std::nearbyint(frac * (1 << f.mbits)));
  if (q == (1 << f.mbits)) { q = 0; e += 1; }
  return s | ((e + f.bias) << f.mbits) | q;
}

/* E8M0 scale byte -> 2^(byte-127); 255 is NaN. */
double e8m0_value(int s) { return s == 255 ? NAN : std::ldexp(1.0, s - 127); }

struct DecodeTables {
  double t[2][256];
  double scale[256];
  DecodeTables() {
    for (int c = 0; c < 256; ++c) {
      t[0][c] = decode(c, kE4M3);
      t[1][c] = decode(c, kE5M2);
      scale[c] = e8m0_value(c);
    }
  }
};
const DecodeTables& tables() { static const DecodeTables d; return d; }

double dequant(uint8_t code, uint8_t scale, int fmt) { return tables().t[fmt][code] * tables().scale[scale]; }

double bf(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t to_bf16(double x) {
  if (std::isnan(x)) return 0x7FC0;
  const uint16_t s = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (a == 0.0) return s;
  if (std::isinf(a)) return s | 0x7F80;
  int ex;
  std::frexp(a, &ex);
  const int e = std::max(ex - 1, -126);             /* bf16 subnormals share 2^-126's quantum */
  const double quantum = std::ldexp(1.0, e - 7);
  const double r = std::nearbyint(a / quantum) * quantum;
  if (r >= 0x1p128) return s | 0x7F80;
  const float rf = float(r);                        /* exact */
  uint32_t u;
  std::memcpy(&u, &rf, 4);
  return s | uint16_t(u >> 16);
}
double bf16r(double x) { return bf(to_bf16(x)); }   /* value after one bf16 rounding   */
double f32r(double x) { return double(float(x)); }  /* value after one fp32 rounding   */
/* A gradient output: the fp64 sum stands for an fp32 accumulator, so it is
 * rounded once to fp32 and then to bf16 (RNE), as an fp32 result would be. */
uint16_t out_bf16(double acc) { return to_bf16(f32r(acc)); }
/* Writes gradient g into an output element: overwritten, or added to the
 * element's value when accumulating (P1's accumulation flag), one rounding. */
void put_grad(uint16_t* o, double g, int accumulate) { *o = out_bf16(accumulate ? bf(*o) + g : g); }

/* One MX group (P1: "32-element quantization group").  Scale rule (reading:
 * the OCP MX rule; the pages do not state one): X = floor(log2(amax)) - emax
 * of the element format, clamped to [-127, 127]; an all-zero group takes
 * X = -127 (byte 0).  Element i is encode(v_i * 2^-X).  Returns the byte. */
int quantize_group(const double* v, int n, int fmt, uint8_t* codes, double* deq) {
  const Fmt* f = fmt_of(fmt);
  if (!f) {                                         /* test hook: no quantisation */
    for (int i = 0; i < n; ++i) { if (codes) codes[i] = 0; if (deq) deq[i] = v[i]; }
    return 127;
  }
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  int X = -127;
  if (amax > 0.0) {
    int ex;
    std::frexp(amax, &ex);
    X = std::min(127, std::max(-127, ex - 1 - f->emax));
  }
  for (int i = 0; i < n; ++i) {
    const int c = encode(std::ldexp(v[i], -X), *f);
    if (codes) codes[i] = uint8_t(c);
    if (deq) deq[i] = std::ldexp(tables().t[fmt][c], X);
  }
  return X + 127;
}

/* Dequantised values of one group taken from a strided source. */
void qgroup_strided(const double* src, int64_t stride, int fmt, double* deq) {
  double v[32];
  for (int k = 0; k < 32; ++k) v[k] = src[k * stride];
  quantize_group(v, 32, fmt, nullptr, deq);
}

int hw_threads(int n) {
  if (n > 0) return n;
  unsigned h = std::thread::hardware_concurrency();
  return h ? int(h) : 1;
}

/* Runs fn(i) for i in [0,n) on nt threads; each index is independent, so the
 * result does not depend on the thread count. */
void parallel_for(int64_t n, int nt, const std::function<void(int64_t)>& fn) {
  nt = int(std::min<int64_t>(hw_threads(nt), std::max<int64_t>(n, 1)));
  if (nt <= 1) { for (int64_t i = 0; i < n; ++i) fn(i); return; }
  std::vector<std::thread> th;
  for (int k = 0; k < nt; ++k)
    th.emplace_back([&, k] { for (int64_t i = k; i < n; i += nt) fn(i); });
  for (auto& t : th) t.join();
}

double silu(double g) { return g / (1.0 + std::exp(-g)); }
double dsilu(double g) {                            /* d/dg [g * sigmoid(g)] */
  const double s = 1.0 / (1.0 + std::exp(-g));
  return s * (1.0 + g * (1.0 - s));
}
/* GELU (reading: the defining form g * Phi(g), Phi the standard normal CDF;
 * P3 names "geglu" as the other gated activation without fixing the GELU
 * form) and its derivative Phi(g) + g * phi(g).  Phi(g) = erfc(-g / sqrt 2) / 2,
 * which keeps its relative accuracy for negative g (1 + erf cancels there). */
double normal_cdf(double g) { return 0.5 * std::erfc(-g / std::sqrt(2.0)); }
double gelu(double g) { return g * normal_cdf(g); }
double dgelu(double g) {
  const double cdf = normal_cdf(g);
  const double pdf = std::exp(-0.5 * g * g) / std::sqrt(2.0 * M_PI);
  return cdf + g * pdf;
}
/* The gate's activation: 0 = SwiGLU (silu), 1 = GeGLU (gelu). */
double act(int a, double g) { return a == 1 ? gelu(g) : silu(g); }
double dact(int a, double g) { return a == 1 ? dgelu(g) : dsilu(g); }

}  // namespace

/* ======================================================================== */
extern "C" {

double orc_fp8_decode(int code, int fmt) { return fmt_of(fmt) ? decode(code & 0xFF, *fmt_of(fmt)) : NAN; }
int orc_fp8_encode(double y, int fmt) { return fmt_of(fmt) ? encode(y, *fmt_of(fmt)) : -1; }
int orc_fp8_encode_array(const double* y, int64_t n, int fmt, uint8_t* out) {
  if (!fmt_of(fmt)) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = uint8_t(encode(y[i], *fmt_of(fmt)));
  return 0;
}
int orc_fp8_emax(int fmt) { return fmt_of(fmt) ? fmt_of(fmt)->emax : -1; }
double orc_bf16_to_double(uint16_t b) { return bf(b); }
uint16_t orc_double_to_bf16(double x) { return to_bf16(x); }

int orc_quantize_group(const double* v, int n, int fmt, uint8_t* codes, double* deq) {
  return quantize_group(v, n, fmt, codes, deq);
}

int orc_quantize(const uint16_t* x, int64_t R, int64_t C, int axis, int fmt, uint8_t* codes,
                 uint8_t* scales) {
  if (!fmt_of(fmt) || R < 0 || C < 0) return -1;
  double v[32];
  uint8_t c[32];
  if (axis == 1) {
    if (C % 32) return -1;
    for (int64_t r = 0; r < R; ++r)
      for (int64_t g = 0; g < C / 32; ++g) {
        for (int k = 0; k < 32; ++k) v[k] = bf(x[r * C + g * 32 + k]);
        scales[r * (C / 32) + g] = uint8_t(quantize_group(v, 32, fmt, c, nullptr));
        for (int k = 0; k < 32; ++k) codes[r * C + g * 32 + k] = c[k];
      }
    return 0;
  }
  if (axis == 0) {
    if (R % 32) return -1;
    for (int64_t g = 0; g < R / 32; ++g)
      for (int64_t col = 0; col < C; ++col) {
        for (int k = 0; k < 32; ++k) v[k] = bf(x[(g * 32 + k) * C + col]);
        scales[g * C + col] = uint8_t(quantize_group(v, 32, fmt, c, nullptr));
        for (int k = 0; k < 32; ++k) codes[(g * 32 + k) * C + col] = c[k];
      }
    return 0;
  }
  return -1;
}

int orc_mx_gemm_nt(const uint8_t* ac, const uint8_t* as, int fa, const uint8_t* bc,
                   const uint8_t* bs, int fb, int64_t M, int64_t N, int64_t K, float* C,
                   int nthreads) {
  if (!fmt_of(fa) || !fmt_of(fb) || K % 32) return -1;
  std::vector<double> A(M * K), B(N * K);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) A[m * K + k] = dequant(ac[m * K + k], as[m * (K / 32) + k / 32], fa);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) B[n * K + k] = dequant(bc[n * K + k], bs[n * (K / 32) + k / 32], fb);
  parallel_for(M, nthreads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += A[m * K + k] * B[n * K + k];
      C[m * N + n] = float(s);
    }
  });
  return 0;
}

/* P2, forward/backward convention: dX = dY @ W (contraction N), dW = dY^T @ X
 * (contraction M).  Reading: each operand is quantised in groups of 32 along
 * the contraction axis of the product it feeds, so dY is quantised twice. */
int orc_dense_bwd(const uint16_t* dY, const uint16_t* W, const uint16_t* X, int64_t M, int64_t N,
                  int64_t K, int fmt_dy, int fmt_w, int fmt_x, const int64_t* dx_rows,
                  int64_t n_dx_rows, uint16_t* dX, const int64_t* dw_rows, int64_t n_dw_rows,
                  uint16_t* dW, int nthreads) {
  if (M % 32 || N % 32 || K < 1) return -1;
  if (dX) {
    /* W quantised along N: groups are columns of 32 consecutive rows of W. */
    std::vector<double> wq(N * K);
    parallel_for(K, nthreads, [&](int64_t k) {
      std::vector<double> col(N);
      for (int64_t n = 0; n < N; ++n) col[n] = bf(W[n * K + k]);
      double d[32];
      for (int64_t g = 0; g < N / 32; ++g) {
        qgroup_strided(&col[g * 32], 1, fmt_w, d);
        for (int k2 = 0; k2 < 32; ++k2) wq[(g * 32 + k2) * K + k] = d[k2];
      }
    });
    const int64_t nr = dx_rows ? n_dx_rows : M;
    parallel_for(nr, nthreads, [&](int64_t r) {
      const int64_t m = dx_rows ? dx_rows[r] : r;
      std::vector<double> row(N), acc(K, 0.0);
      for (int64_t n = 0; n < N; ++n) row[n] = bf(dY[m * N + n]);
      std::vector<double> q(N);
      for (int64_t g = 0; g < N / 32; ++g) qgroup_strided(&row[g * 32], 1, fmt_dy, &q[g * 32]);
      for (int64_t n = 0; n < N; ++n) {
        const double c = q[n];
        const double* w = &wq[n * K];
        for (int64_t k = 0; k < K; ++k) acc[k] += c * w[k];
      }
      for (int64_t k = 0; k < K; ++k) dX[r * K + k] = out_bf16(acc[k]);
    });
  }
  if (dW) {
    /* X quantised along M (groups of 32 consecutive rows per column). */
    std::vector<double> xq(M * K);
    parallel_for(K, nthreads, [&](int64_t k) {
      std::vector<double> col(M);
      for (int64_t m = 0; m < M; ++m) col[m] = bf(X[m * K + k]);
      double d[32];
      for (int64_t g = 0; g < M / 32; ++g) {
        qgroup_strided(&col[g * 32], 1, fmt_x, d);
        for (int k2 = 0; k2 < 32; ++k2) xq[(g * 32 + k2) * K + k] = d[k2];
      }
    });
    const int64_t nr = dw_rows ? n_dw_rows : N;
    parallel_for(nr, nthreads, [&](int64_t r) {
      const int64_t n = dw_rows ? dw_rows[r] : r;
      std::vector<double> col(M), q(M), acc(K, 0.0);
      for (int64_t m = 0; m < M; ++m) col[m] = bf(dY[m * N + n]);   /* dY quantised along M */
      for (int64_t g = 0; g < M / 32; ++g) qgroup_strided(&col[g * 32], 1, fmt_dy, &q[g * 32]);
      for (int64_t m = 0; m < M; ++m) {
        const double c = q[m];
        const double* x = &xq[m * K];
        for (int64_t k = 0; k < K; ++k) acc[k] += c * x[k];
      }
      for (int64_t k = 0; k < K; ++k) dW[r * K + k] = out_bf16(acc[k]);
    });
  }
  return 0;
}

/* P1 "Dimensions": N = (T*TopK - (E-1))/B + E - 1, read with "/" as ceiling
 * division: the worst case of sum_e ceil(n_e/B) over all loads n_e >= 0 with
 * sum n_e = T*TopK, which equals E + floor((T*TopK - E)/B) for T*TopK >= E. */
int64_t orc_num_blocks(int64_t T, int64_t K, int64_t E, int64_t B) {
  const int64_t num = T * K - (E - 1);
  if (B <= 0 || E <= 0 || T * K < E) return -1;   /* fewer pairs than experts: not covered */
  return (num + B - 1) / B + E - 1;
}

/* Reading of the block layout (P1 gives the tensors, not their construction):
 * experts in ascending id, each owning ceil(n_e/B) consecutive blocks; inside
 * an expert, tokens in ascending id; the tail of an expert's last block and
 * every trailing unused block hold -1; unused blocks map to expert E-1. */
int orc_build_blocks(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B, int64_t N,
                     int32_t* tpid, int32_t* b2e) {
  std::vector<std::vector<int32_t>> tok(E);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t k = 0; k < K; ++k) {
      const int32_t e = topk[t * K + k];
      if (e < 0) continue;   // a dropped selection: this token has fewer than K experts
      if (e >= E) return -1;
      tok[e].push_back(int32_t(t));
    }
  int64_t need = 0;
  for (int64_t e = 0; e < E; ++e) need += (int64_t(tok[e].size()) + B - 1) / B;
  if (need > N) return -1;
  for (int64_t s = 0; s < N * B; ++s) tpid[s] = -1;
  for (int64_t b = 0; b < N; ++b) b2e[b] = int32_t(E - 1);
  int64_t blk = 0;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t nb = (int64_t(tok[e].size()) + B - 1) / B;
    for (size_t j = 0; j < tok[e].size(); ++j) tpid[blk * B + int64_t(j)] = tok[e][j];
    for (int64_t q = 0; q < nb; ++q) b2e[blk + q] = int32_t(e);
    blk += nb;
  }
  return 0;
}

}  // extern "C"

/* ======================================================================== */
/* MoE backward in MXFP8 mode.                                               */
namespace {

struct Moe {
  const orc_moe_problem& p;
  explicit Moe(const orc_moe_problem& pp) : p(pp) {}

  /* dequantised weights, groups along the backward contraction axis:
   * W_down[e][i][:] along H, W_gate_up[e][h][j][:] along I. */
  double wd(int64_t e, int64_t i, int64_t h) const {
    const int64_t r = e * p.I + i;
    return dequant(p.wd_codes[r * p.H + h], p.wd_scales[r * (p.H / 32) + h / 32], p.fmt_w);
  }
  double wgu(int64_t e, int64_t h, int j, int64_t i) const {
    const int64_t r = (e * p.H + h) * 2 + j;
    return dequant(p.wgu_codes[r * p.I + i], p.wgu_scales[r * (p.I / 32) + i / 32], p.fmt_w);
  }
  int64_t token(int64_t b, int64_t s) const {
    const int64_t t = p.tpid[b * p.B + s];
    return (t >= 0 && t < p.T) ? t : -1;             /* outside [0,T) = padding slot */
  }
  double affinity(int64_t t, int64_t e) const { return t < 0 ? 0.0 : double(p.aff[t * p.E + e]); }
  double dy(int64_t t, int64_t h) const { return t < 0 ? 0.0 : bf(p.dy[t * p.H + h]); }
  double x(int64_t t, int64_t h) const { return t < 0 ? 0.0 : bf(p.hidden[t * p.H + h]); }
  /* P1 gate_up_proj_act_checkpoint_T [N,2,I,B]: [b,0] = gate_pre, [b,1] = up.
   * Reading: a padding slot's checkpoint content is ignored (taken as 0). */
  double ckpt(int64_t b, int j, int64_t i, int64_t s, int64_t t) const {
    return t < 0 ? 0.0 : bf(p.ckpt[((b * 2 + j) * p.I + i) * p.B + s]);
  }

  /* Phase-1 operand: dY row of token t quantised along H (fmt_grad). */
  void dy_row_q(int64_t t, std::vector<double>& q) const {
    q.assign(p.H, 0.0);
    if (t < 0) return;
    std::vector<double> row(p.H);
    for (int64_t h = 0; h < p.H; ++h) row[h] = dy(t, h);
    for (int64_t g = 0; g < p.H / 32; ++g) qgroup_strided(&row[g * 32], 1, p.fmt_grad, &q[g * 32]);
  }

  /* Per-slot epilogue values at intermediate column i (P1 "SwiGLU recompute"
   * of gate_act and intermediate from the checkpoint; P3
   * _down_projection_backward_act: gated-activation backward with the row
   * scale and the row reduction).  Rounding points (reading): gate_act and
   * intermediate are bf16, as P1 lets the caller supply them; dS and dInter
   * are fp32; dGate and dUp are rounded to bf16 before any quantisation. */
  struct Col { double g, u, ga, inter, dS, dG, dU; };
  Col col(int64_t b, int64_t s, int64_t t, int64_t e, int64_t i, const std::vector<double>& dyq) const {
    Col c;
    c.g = ckpt(b, 0, i, s, t);
    c.u = ckpt(b, 1, i, s, t);
    c.ga = bf16r(act(p.activation, c.g));
    c.inter = bf16r(c.ga * c.u);
    double acc = 0.0;                                /* Phase 1: dS = Q(dY_t) . Q(W_down[e][i]) */
    for (int64_t h = 0; h < p.H; ++h) acc += dyq[h] * wd(e, i, h);
    c.dS = f32r(acc);
    const double dinter = f32r(affinity(t, e) * c.dS);   /* affinity applied to the fp32 tile */
    c.dG = bf16r(dinter * c.u * dact(p.activation, c.g));
    c.dU = bf16r(dinter * c.ga);
    return c;
  }

  /* Bias part of d(affinity): <dY_t, b2[e]> (P3 db2_and_ds_kernel). */
  double bias_dot(int64_t t, int64_t e) const {
    if (!p.has_bias || !p.b2 || t < 0) return 0.0;
    double s = 0.0;
    for (int64_t h = 0; h < p.H; ++h) s += dy(t, h) * bf(p.b2[e * p.H + h]);
    return s;
  }

  /* Full row of one slot: dG, dU over all I, and d(affinity) =
   * sum_i dS*intermediate + <dY, b2> (P3: colvec_reduce of the GEMM plus the
   * bias term).  Returns d(affinity) unrounded. */
  double slot_row(int64_t b, int64_t s, std::vector<double>* dS, std::vector<double>* ga,
                  std::vector<double>* inter, std::vector<double>& dG, std::vector<double>& dU) const {
    const int64_t t = token(b, s), e = p.b2e[b];
    std::vector<double> dyq;
    dy_row_q(t, dyq);
    dG.assign(p.I, 0.0);
    dU.assign(p.I, 0.0);
    if (dS) dS->assign(p.I, 0.0);
    if (ga) ga->assign(p.I, 0.0);
    if (inter) inter->assign(p.I, 0.0);
    double daff = 0.0;
    for (int64_t i = 0; i < p.I; ++i) {
      const Col c = col(b, s, t, e, i, dyq);
      daff += c.dS * c.inter;
      dG[i] = c.dG;
      dU[i] = c.dU;
      if (dS) (*dS)[i] = c.dS;
      if (ga) (*ga)[i] = c.ga;
      if (inter) (*inter)[i] = c.inter;
    }
    return daff + bias_dot(t, e);
  }

  /* Phase 3 for one slot: Q_I([dG, dU]) . Q(W_gate_up[e])^T, added into acc[H]
   * (fp64).  dGate and dUp are quantised separately, in groups along I. */
  void phase3(int64_t e, const std::vector<double>& dG, const std::vector<double>& dU,
              std::vector<double>& acc) const {
    std::vector<double> q[2] = {std::vector<double>(p.I), std::vector<double>(p.I)};
    for (int64_t g = 0; g < p.I / 32; ++g) {
      qgroup_strided(&dG[g * 32], 1, p.fmt_grad, &q[0][g * 32]);
      qgroup_strided(&dU[g * 32], 1, p.fmt_grad, &q[1][g * 32]);
    }
    for (int64_t h = 0; h < p.H; ++h) {
      double s = 0.0;
      for (int j = 0; j < 2; ++j)
        for (int64_t i = 0; i < p.I; ++i) s += q[j][i] * wgu(e, h, j, i);
      acc[h] += s;
    }
  }
};

bool valid_problem(const orc_moe_problem* p) {
  return p && p->T > 0 && p->H % 32 == 0 && p->I % 32 == 0 && p->B % 32 == 0 && p->E > 0 &&
         (p->activation == 0 || p->activation == 1) &&
         p->N > 0 && fmt_of(p->fmt_w) && (fmt_of(p->fmt_act) || p->fmt_act == -1) &&
         (fmt_of(p->fmt_grad) || p->fmt_grad == -1);
}

}  // namespace

extern "C" {

int orc_moe_token_rows(const orc_moe_problem* pp, const int32_t* tokens, int64_t ntok,
                       uint16_t* dx_rows, uint16_t* daff_rows) {
  if (!valid_problem(pp)) return -1;
  const Moe m(*pp);
  const orc_moe_problem& p = *pp;
  parallel_for(ntok, p.nthreads, [&](int64_t r) {
    const int64_t t = tokens[r];
    std::vector<double> acc(p.H, 0.0), daff(p.E, 0.0), dG, dU;
    for (int64_t b = 0; b < p.N; ++b)
      for (int64_t s = 0; s < p.B; ++s) {
        if (m.token(b, s) != t || t < 0) continue;
        const int64_t e = p.b2e[b];
        daff[e] += m.slot_row(b, s, nullptr, nullptr, nullptr, dG, dU);
        m.phase3(e, dG, dU, acc);
      }
    if (dx_rows)
      for (int64_t h = 0; h < p.H; ++h) put_grad(&dx_rows[r * p.H + h], acc[h], p.accumulate);
    if (daff_rows)
      for (int64_t e = 0; e < p.E; ++e) put_grad(&daff_rows[r * p.E + e], daff[e], p.accumulate);
  });
  return 0;
}

/* Phases 2 and 4 and the bias gradients for one expert (P1: dW_gate_up and
 * dW_down, reduced over the expert's blocks; P3 _up_projection_backward_weight,
 * _down_projection_backward_weight, db1_kernel, db2_and_ds_kernel).  The
 * token-axis operands are quantised in groups of 32 consecutive slots of one
 * block (reading: the contraction axis of these products is the token axis).
 *   dW_gate_up[e][h][j][i] = sum_slots Q_act(X)[s][h] * Q_grad([dG,dU])[s][j][i]
 *   on H: dW_down[e][i][h] = sum_slots Q_act(inter)[s][i] * Q_grad(bf16(a*dY))[s][h]
 *   on I: dW_down[e][i][h] = sum_slots Q_act(bf16(a*inter))[s][i] * Q_grad(dY)[s][h]
 *   db1[e][j][i] = sum_slots [dG,dU][s][j][i];  db2[e][h] = sum_slots a*dY[s][h]. */
int orc_moe_expert_cols(const orc_moe_problem* pp, int64_t e, const int32_t* icols, int64_t nicol,
                        uint16_t* dwgu_cols, uint16_t* dwd_rows, uint16_t* db1_cols,
                        uint16_t* db2_row) {
  if (!valid_problem(pp) || e < 0 || e >= pp->E) return -1;
  const Moe m(*pp);
  const orc_moe_problem& p = *pp;
  std::vector<int64_t> blocks;
  for (int64_t b = 0; b < p.N; ++b)
    if (p.b2e[b] == e) blocks.push_back(b);
  const int64_t S = int64_t(blocks.size()) * p.B;
  const int64_t C = nicol;
  std::vector<int64_t> tok(S);
  std::vector<double> a(S);
  for (int64_t q = 0; q < S; ++q) {
    tok[q] = m.token(blocks[q / p.B], q % p.B);
    a[q] = m.affinity(tok[q], e);
  }
  /* per slot and selected column: dG, dU and the Phase-4 activation operand */
  std::vector<double> gv(S * C), uv(S * C), iv(S * C);
  parallel_for(S, p.nthreads, [&](int64_t q) {
    const int64_t b = blocks[q / p.B], s = q % p.B;
    std::vector<double> dyq;
    m.dy_row_q(tok[q], dyq);
    for (int64_t c = 0; c < C; ++c) {
      const Moe::Col v = m.col(b, s, tok[q], e, icols[c], dyq);
      gv[q * C + c] = v.dG;
      uv[q * C + c] = v.dU;
      iv[q * C + c] = p.affinity_on == 1 ? bf16r(f32r(a[q] * v.inter)) : v.inter;
    }
  });
  /* quantise the per-column operands along slots */
  std::vector<double> gq(S * C), uq(S * C), iq(S * C);
  for (int64_t g = 0; g < S / 32; ++g)
    for (int64_t c = 0; c < C; ++c) {
      double d[32];
      qgroup_strided(&gv[g * 32 * C + c], C, p.fmt_grad, d);
      for (int k = 0; k < 32; ++k) gq[(g * 32 + k) * C + c] = d[k];
      qgroup_strided(&uv[g * 32 * C + c], C, p.fmt_grad, d);
      for (int k = 0; k < 32; ++k) uq[(g * 32 + k) * C + c] = d[k];
      qgroup_strided(&iv[g * 32 * C + c], C, p.fmt_act, d);
      for (int k = 0; k < 32; ++k) iq[(g * 32 + k) * C + c] = d[k];
    }
  if (db1_cols)
    for (int64_t c = 0; c < C; ++c) {
      double s0 = 0.0, s1 = 0.0;
      for (int64_t q = 0; q < S; ++q) { s0 += gv[q * C + c]; s1 += uv[q * C + c]; }
      put_grad(&db1_cols[c], s0, p.accumulate);
      put_grad(&db1_cols[C + c], s1, p.accumulate);
    }
  parallel_for(p.H, p.nthreads, [&](int64_t h) {
    std::vector<double> xs(S), ys(S), xq(S), yq(S);
    double db2 = 0.0;
    for (int64_t q = 0; q < S; ++q) {
      const double dyv = m.dy(tok[q], h);
      xs[q] = m.x(tok[q], h);
      /* on H: bf16(fp32(a*dY)) (P1 down_proj_act_checkpoint = output_grad * affinity) */
      ys[q] = p.affinity_on == 1 ? dyv : bf16r(f32r(a[q] * dyv));
      db2 += a[q] * dyv;
    }
    for (int64_t g = 0; g < S / 32; ++g) {
      qgroup_strided(&xs[g * 32], 1, p.fmt_act, &xq[g * 32]);
      qgroup_strided(&ys[g * 32], 1, p.fmt_grad, &yq[g * 32]);
    }
    for (int64_t c = 0; c < C; ++c) {
      double s0 = 0.0, s1 = 0.0, s2 = 0.0;
      for (int64_t q = 0; q < S; ++q) {
        s0 += xq[q] * gq[q * C + c];
        s1 += xq[q] * uq[q * C + c];
        s2 += iq[q * C + c] * yq[q];
      }
      if (dwgu_cols) {
        put_grad(&dwgu_cols[(h * 2 + 0) * C + c], s0, p.accumulate);
        put_grad(&dwgu_cols[(h * 2 + 1) * C + c], s1, p.accumulate);
      }
      if (dwd_rows) put_grad(&dwd_rows[c * p.H + h], s2, p.accumulate);
    }
    if (db2_row) put_grad(&db2_row[h], db2, p.accumulate);
  });
  return 0;
}

int orc_moe_bwd(const orc_moe_problem* pp, uint16_t* dx, uint16_t* daff, uint16_t* dwgu,
                uint16_t* dwd, uint16_t* db1, uint16_t* db2) {
  if (!valid_problem(pp)) return -1;
  const orc_moe_problem& p = *pp;
  std::vector<int32_t> all_t(p.T);
  for (int64_t t = 0; t < p.T; ++t) all_t[t] = int32_t(t);
  std::vector<uint16_t> daff_rows(p.T * p.E);
  if (p.accumulate && daff) std::memcpy(daff_rows.data(), daff, daff_rows.size() * 2);
  if (orc_moe_token_rows(pp, all_t.data(), p.T, dx, daff_rows.data())) return -1;
  if (daff) std::memcpy(daff, daff_rows.data(), daff_rows.size() * 2);
  std::vector<int32_t> all_i(p.I);
  for (int64_t i = 0; i < p.I; ++i) all_i[i] = int32_t(i);
  for (int64_t e = 0; e < p.E; ++e) {
    const int rc = orc_moe_expert_cols(pp, e, all_i.data(), p.I, dwgu ? dwgu + e * p.H * 2 * p.I : nullptr,
                                       dwd ? dwd + e * p.I * p.H : nullptr, db1 ? db1 + e * 2 * p.I : nullptr,
                                       db2 ? db2 + e * p.H : nullptr);
    if (rc) return rc;
  }
  return 0;
}

int orc_moe_block_detail(const orc_moe_problem* pp, int64_t b, float* dS, uint16_t* ga,
                         uint16_t* inter, uint16_t* dG, uint16_t* dU, float* daff_slot) {
  if (!valid_problem(pp) || b < 0 || b >= pp->N) return -1;
  const Moe m(*pp);
  const orc_moe_problem& p = *pp;
  parallel_for(p.B, p.nthreads, [&](int64_t s) {
    std::vector<double> vs, vga, vin, vg, vu;
    const double da = m.slot_row(b, s, &vs, &vga, &vin, vg, vu);
    for (int64_t i = 0; i < p.I; ++i) {
      if (dS) dS[s * p.I + i] = float(vs[i]);
      if (ga) ga[s * p.I + i] = to_bf16(vga[i]);
      if (inter) inter[s * p.I + i] = to_bf16(vin[i]);
      if (dG) dG[s * p.I + i] = to_bf16(vg[i]);
      if (dU) dU[s * p.I + i] = to_bf16(vu[i]);
    }
    if (daff_slot) daff_slot[s] = float(da);
  });
  return 0;
}

int orc_moe_token_operand(const orc_moe_problem* pp, int which, uint8_t* codes, uint8_t* scales) {
  if (!valid_problem(pp) || which < 0 || which > 3) return -1;
  const Moe m(*pp);
  const orc_moe_problem& p = *pp;
  const int64_t P = p.N * p.B;
  const int64_t rows = which <= 1 ? p.H : (which == 2 ? p.I : 2 * p.I);
  const int fmt = (which == 0 || which == 2) ? p.fmt_act : p.fmt_grad;
  std::vector<double> val(rows * P, 0.0);            /* [rows][P] values before quantisation */
  parallel_for(p.N, p.nthreads, [&](int64_t b) {
    const int64_t e = p.b2e[b];
    for (int64_t s = 0; s < p.B; ++s) {
      const int64_t t = m.token(b, s), q = b * p.B + s;
      const double a = m.affinity(t, e);
      if (which == 0)
        for (int64_t h = 0; h < p.H; ++h) val[h * P + q] = m.x(t, h);
      else if (which == 1)
        for (int64_t h = 0; h < p.H; ++h)
          val[h * P + q] = p.affinity_on == 1 ? m.dy(t, h) : bf16r(f32r(a * m.dy(t, h)));
      else {
        std::vector<double> vin, vg, vu;
        m.slot_row(b, s, nullptr, nullptr, &vin, vg, vu);
        for (int64_t i = 0; i < p.I; ++i) {
          if (which == 2) val[i * P + q] = p.affinity_on == 1 ? bf16r(f32r(a * vin[i])) : vin[i];
          else { val[i * P + q] = vg[i]; val[(p.I + i) * P + q] = vu[i]; }
        }
      }
    }
  });
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < P / 32; ++g) {
      uint8_t c[32];
      scales[r * (P / 32) + g] = uint8_t(quantize_group(&val[r * P + g * 32], 32, fmt, c, nullptr));
      std::memcpy(&codes[r * P + g * 32], c, 32);
    }
  return 0;
}

/* ======================================================================== */
/* Exact mode: the plain definition of the layer and its gradients in fp64.
 * Forward per routed slot (block b with expert e, token t, affinity a):
 *   g = x_t W_gu[e][:,0,:] + b1[e,0],  u = x_t W_gu[e][:,1,:] + b1[e,1]
 *   inter = act(g) * u     (act = silu for SwiGLU, gelu for GeGLU)
 *   on H: y_t += a * (inter W_down[e] + b2[e])
 *   on I: y_t += (a * inter) W_down[e]                                        */
int orc_moe_fwd_exact(const orc_moe_exact_problem* p, double* y, double* gu_ckpt) {
  const int64_t T = p->T, H = p->H, I = p->I, E = p->E;
  std::fill(y, y + T * H, 0.0);
  if (gu_ckpt) std::fill(gu_ckpt, gu_ckpt + p->N * 2 * I * p->B, 0.0);
  std::vector<double> g(I), u(I);
  for (int64_t b = 0; b < p->N; ++b)
    for (int64_t s = 0; s < p->B; ++s) {
      const int64_t t = p->tpid[b * p->B + s];
      if (t < 0 || t >= T) continue;
      const int64_t e = p->b2e[b];
      const double a = p->aff[t * E + e];
      for (int64_t i = 0; i < I; ++i) {
        double sg = p->b1 ? p->b1[(e * 2 + 0) * I + i] : 0.0;
        double su = p->b1 ? p->b1[(e * 2 + 1) * I + i] : 0.0;
        for (int64_t h = 0; h < H; ++h) {
          sg += p->x[t * H + h] * p->wgu[((e * H + h) * 2 + 0) * I + i];
          su += p->x[t * H + h] * p->wgu[((e * H + h) * 2 + 1) * I + i];
        }
        g[i] = sg;
        u[i] = su;
        if (gu_ckpt) {
          gu_ckpt[((b * 2 + 0) * I + i) * p->B + s] = sg;
          gu_ckpt[((b * 2 + 1) * I + i) * p->B + s] = su;
        }
      }
      for (int64_t h = 0; h < H; ++h) {
        double d = 0.0;
        for (int64_t i = 0; i < I; ++i) d += act(p->activation, g[i]) * u[i] * p->wd[(e * I + i) * H + h];
        if (p->affinity_on == 1) y[t * H + h] += a * d;
        else y[t * H + h] += a * (d + (p->b2 ? p->b2[e * H + h] : 0.0));
      }
    }
  return 0;
}

/* Gradients of L = <dY, y> (P1's return tuple; the bias-gradient forms follow
 * P3's db1_kernel and db2_and_ds_kernel):
 *   d(a)      = <dY_t, inter W_down[e] + b2[e]>
 *   dInter    = a * (dY_t W_down[e]^T)
 *   dG        = dInter * u * act'(g),  dU = dInter * act(g)
 *   dX_t     += [dG, dU] W_gu[e]^T
 *   dW_gu[e] += x_t^T [dG, dU],  dW_down[e] += inter^T (a dY_t)
 *   db1[e]   += [dG, dU],        db2[e]     += a dY_t                        */
int orc_moe_bwd_exact(const orc_moe_exact_problem* p, const double* dy, double* dx, double* daff,
                      double* dwgu, double* dwd, double* db1, double* db2) {
  const int64_t T = p->T, H = p->H, I = p->I, E = p->E;
  std::fill(dx, dx + T * H, 0.0);
  std::fill(daff, daff + T * E, 0.0);
  std::fill(dwgu, dwgu + E * H * 2 * I, 0.0);
  std::fill(dwd, dwd + E * I * H, 0.0);
  if (db1) std::fill(db1, db1 + E * 2 * I, 0.0);
  if (db2) std::fill(db2, db2 + E * H, 0.0);
  std::vector<double> g(I), u(I), inter(I), dS(I), dG(I), dU(I);
  for (int64_t b = 0; b < p->N; ++b)
    for (int64_t s = 0; s < p->B; ++s) {
      const int64_t t = p->tpid[b * p->B + s];
      if (t < 0 || t >= T) continue;
      const int64_t e = p->b2e[b];
      const double a = p->aff[t * E + e];
      for (int64_t i = 0; i < I; ++i) {
        double sg = p->b1 ? p->b1[(e * 2 + 0) * I + i] : 0.0;
        double su = p->b1 ? p->b1[(e * 2 + 1) * I + i] : 0.0;
        for (int64_t h = 0; h < H; ++h) {
          sg += p->x[t * H + h] * p->wgu[((e * H + h) * 2 + 0) * I + i];
          su += p->x[t * H + h] * p->wgu[((e * H + h) * 2 + 1) * I + i];
        }
        g[i] = sg;
        u[i] = su;
        inter[i] = act(p->activation, sg) * su;
        double d = 0.0;
        for (int64_t h = 0; h < H; ++h) d += dy[t * H + h] * p->wd[(e * I + i) * H + h];
        dS[i] = d;
      }
      double da = 0.0;
      for (int64_t i = 0; i < I; ++i) da += inter[i] * dS[i];
      if (p->b2)
        for (int64_t h = 0; h < H; ++h) da += dy[t * H + h] * p->b2[e * H + h];
      daff[t * E + e] += da;
      for (int64_t i = 0; i < I; ++i) {
        const double dinter = a * dS[i];
        dG[i] = dinter * u[i] * dact(p->activation, g[i]);
        dU[i] = dinter * act(p->activation, g[i]);
      }
      for (int64_t h = 0; h < H; ++h) {
        double sx = 0.0;
        for (int64_t i = 0; i < I; ++i)
          sx += dG[i] * p->wgu[((e * H + h) * 2 + 0) * I + i] + dU[i] * p->wgu[((e * H + h) * 2 + 1) * I + i];
        dx[t * H + h] += sx;
        for (int64_t i = 0; i < I; ++i) {
          dwgu[((e * H + h) * 2 + 0) * I + i] += p->x[t * H + h] * dG[i];
          dwgu[((e * H + h) * 2 + 1) * I + i] += p->x[t * H + h] * dU[i];
        }
      }
      for (int64_t i = 0; i < I; ++i)
        for (int64_t h = 0; h < H; ++h) dwd[(e * I + i) * H + h] += inter[i] * a * dy[t * H + h];
      if (db1)
        for (int64_t i = 0; i < I; ++i) { db1[(e * 2 + 0) * I + i] += dG[i]; db1[(e * 2 + 1) * I + i] += dU[i]; }
      if (db2)
        for (int64_t h = 0; h < H; ++h) db2[e * H + h] += a * dy[t * H + h];
    }
  return 0;
}

}  // extern "C"
