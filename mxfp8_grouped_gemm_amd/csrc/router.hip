// router.hip -- the router backward that consumes the affinity gradient (P3,
// sonic-moe functional/backward.py: the softmax-over-top-k, top-k-over-softmax
// and top-k scatter backward kernels).
//
// Per token t with selected experts idx[t][0..K) and upstream score gradients
// g[t][k] (given [T,K] in fp32, or read from an affinity gradient laid out
// [T,E] in bf16 at idx), the logit gradient d[t][0..E):
//   softmax over top-k   (scores y = softmax of the K selected logits):
//     d[idx_k] = y_k (g_k - sum_m g_m y_m); 0 elsewhere.
//   top-k over softmax   (p = softmax of all E logits, scores p[idx_k], or
//                         p[idx_k] / S with S = sum_k p[idx_k] when renormalised):
//     dp_k = g_k, or (g_k - sum_m g_m s_m) / S renormalised;
//     d[e] = p_e (dp(e) - sum_k dp_k p[idx_k]), dp(e) = dp_k at e = idx_k, else 0.
//   top-k scatter        (scores = the selected logits): d[idx_k] = g_k; 0 elsewhere.
// Every d[t][e] is written.  HBM-bound: a row is E fp32 logits read (top-k over
// softmax only) and E fp32 gradients written, plus the K selections.
//
// Layout of the work: L lanes take one row (L = E/8 rounded to a power of two
// in [8, 64]), so a wave holds 64 / L rows and each lane EPL = E/L <= 8 of the
// row's columns, lane, lane + L, ..., in registers: a row's loads and stores
// are contiguous across its lanes and issue together, and the row's
// reductions are butterflies over its L lanes.  (One 64-lane wave per row ran
// the fine workload's router at 9-14% of HBM bandwidth: four rounds of waves,
// each waiting on its row's chain of dependent loads.)  Rows wider than
// 64 * 8 columns loop over their columns instead.
#include "kernels.hpp"
#include "mx_device.hpp"

namespace mx {

namespace {
constexpr int kRouterThreads = 256;

template <int L>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int o = 1; o < L; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int L>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}
}  // namespace

template <int L, int EPL, int MODE, bool RENORM, bool DAFF>
__global__ void __launch_bounds__(kRouterThreads) router_bwd_kernel(RouterArgs p) {
  const int lane = threadIdx.x % L;
  const int64_t t = int64_t(blockIdx.x) * (kRouterThreads / L) + threadIdx.x / L;
  if (t >= p.T) return;   // whole segments leave together, so the butterflies stay in step
  const int E = int(p.E), K = int(p.K);
  const int32_t* idx = p.idx + t * K;
  float* out = p.dlogits + t * p.E;
  // upstream gradient of selection k (0 for an index outside [0, E))
  auto grad = [&](int k) -> float {
    const int e = idx[k];
    if (e < 0 || e >= E) return 0.f;
    return DAFF ? bf16_to_f32(p.daff[t * p.E + e]) : p.dscores[t * K + k];
  };
  // columns of this lane: lane + L * j (j < EPL), or a loop when EPL == 0
  constexpr int NJ = EPL > 0 ? EPL : 1;
  if (MODE == kRouterSoftmaxOverTopk || MODE == kRouterTopk) {
    float dot = 0.f;
    if (MODE == kRouterSoftmaxOverTopk)
      for (int k = 0; k < K; ++k) dot += grad(k) * p.scores[t * K + k];
    // value at column e: selection k's term when e = idx[k], else 0
    auto value = [&](int e) -> float {
      float v = 0.f;
      for (int k = 0; k < K; ++k)
        if (idx[k] == e) v = MODE == kRouterTopk ? grad(k) : p.scores[t * K + k] * (grad(k) - dot);
      return v;
    };
    if (EPL > 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + L * j;
        if (e < E) out[e] = value(e);
      }
    } else {
      for (int e = lane; e < E; e += L) out[e] = value(e);
    }
  } else {   // top-k over softmax
    const float* z = p.logits + t * p.E;
    float zv[NJ];
    float m = -INFINITY;
    if (EPL > 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + L * j;
        zv[j] = e < E ? z[e] : -INFINITY;
        m = fmaxf(m, zv[j]);
      }
    } else {
      for (int e = lane; e < E; e += L) m = fmaxf(m, z[e]);
    }
    m = seg_max<L>(m);
    float s = 0.f;
    if (EPL > 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        zv[j] = lane + L * j < E ? expf(zv[j] - m) : 0.f;   // unnormalised probabilities
        s += zv[j];
      }
    } else {
      for (int e = lane; e < E; e += L) s += expf(z[e] - m);
    }
    s = seg_sum<L>(s);
    const float inv_s = 1.f / s;
    // the selected probabilities and the adjusted gradients at them
    float psum = 0.f, gdot = 0.f;
    for (int k = 0; k < K; ++k) {
      const int e = idx[k];
      if (e < 0 || e >= E) continue;
      psum += expf(z[e] - m) * inv_s;
      if (RENORM) gdot += grad(k) * p.scores[t * K + k];
    }
    const float inv_psum = RENORM ? 1.f / psum : 1.f;
    float dot = 0.f;   // sum_k dp_k p[idx_k]
    for (int k = 0; k < K; ++k) {
      const int e = idx[k];
      if (e < 0 || e >= E) continue;
      const float dpk = RENORM ? (grad(k) - gdot) * inv_psum : grad(k);
      dot += dpk * (expf(z[e] - m) * inv_s);
    }
    auto dp_at = [&](int e) -> float {
      float dp = 0.f;
      for (int k = 0; k < K; ++k)
        if (idx[k] == e) dp = RENORM ? (grad(k) - gdot) * inv_psum : grad(k);
      return dp;
    };
    if (EPL > 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + L * j;
        if (e < E) out[e] = zv[j] * inv_s * (dp_at(e) - dot);
      }
    } else {
      for (int e = lane; e < E; e += L) out[e] = expf(z[e] - m) * inv_s * (dp_at(e) - dot);
    }
  }
}

template <int L, int EPL, int MODE>
static void router_go(const RouterArgs& p, unsigned grid, hipStream_t st) {
  if (MODE == kRouterTopkOverSoftmax && p.renorm) {
    if (p.daff) router_bwd_kernel<L, EPL, MODE, true, true><<<grid, kRouterThreads, 0, st>>>(p);
    else router_bwd_kernel<L, EPL, MODE, true, false><<<grid, kRouterThreads, 0, st>>>(p);
  } else {
    if (p.daff) router_bwd_kernel<L, EPL, MODE, false, true><<<grid, kRouterThreads, 0, st>>>(p);
    else router_bwd_kernel<L, EPL, MODE, false, false><<<grid, kRouterThreads, 0, st>>>(p);
  }
}

template <int L, int EPL>
static void router_mode(const RouterArgs& p, hipStream_t st) {
  const int64_t rows_per_wg = kRouterThreads / L;
  const unsigned grid = unsigned((p.T + rows_per_wg - 1) / rows_per_wg);
  if (p.mode == kRouterSoftmaxOverTopk) router_go<L, EPL, kRouterSoftmaxOverTopk>(p, grid, st);
  else if (p.mode == kRouterTopkOverSoftmax) router_go<L, EPL, kRouterTopkOverSoftmax>(p, grid, st);
  else router_go<L, EPL, kRouterTopk>(p, grid, st);
}

hipError_t launch_router_bwd(const RouterArgs& p, hipStream_t st) {
  if (p.T <= 0) return hipSuccess;
  if ((p.T + 3) / 4 > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  // L = E/8 rounded up to a power of two, kept in [8, 64]; EPL = columns per lane
  if (p.E <= 8) router_mode<8, 1>(p, st);
  else if (p.E <= 16) router_mode<8, 2>(p, st);
  else if (p.E <= 32) router_mode<8, 4>(p, st);
  else if (p.E <= 64) router_mode<8, 8>(p, st);
  else if (p.E <= 128) router_mode<16, 8>(p, st);
  else if (p.E <= 256) router_mode<32, 8>(p, st);
  else if (p.E <= 512) router_mode<64, 8>(p, st);
  else router_mode<64, 0>(p, st);
  return hipGetLastError();
}

}  // namespace mx
