// moe_gemm.hip -- the token-block GEMMs of the MoE backward with their fused
// epilogues (P1, "Blockwise MM Backward MXFP8 Kernel API Reference": Phases
// 1 and 3; P3, sonic-moe functional/backward.py: _down_projection_backward_act
// and _up_projection_backward_act).
//
// Phase 1, per block b of expert e (tile rows = intermediate index i,
// tile columns = block slot p, contraction over H; the operands are the
// exactly dequantised MX values in bf16, reduced with bf16 MFMAs whose fp32
// accumulation is exact enough that requantising the result below makes the
// same rounding decisions as an exact sum would):
//   dS[i][p]   = sum_h deq(W_down[e])[i][h] * deq(dY[tok_p])[h]   (dY rows are
//                quantised along H once and gathered here by token id)
//   epilogue:  ga = bf16(silu(g)), inter = bf16(ga*u)   (g,u from the checkpoint)
//              d(a)_p += sum_i dS*inter                  (fp32 atomics per slot)
//              dInter = a_p * dS
//              dGate = bf16(dInter*u*silu'(g)), dUp = bf16(dInter*ga)
//              -> quantised along I (Phase-3 A operand, [P][2I])
//              -> quantised along the slots (Phase-2 B operand, [2I][P])
//              -> db1 partial sums (with a bias)
// Phase 3, per block b (tile rows = slot p, columns = hidden index h,
// contraction over 2I):
//   dX[tok_p][h] += sum_{j,i} deq(dGU)[p][j][i] * deq(W_gate_up[e])[h][j][i]
//   as fp32 atomic adds (a token's top-k slots sit in different blocks).
#include "gemm_v2.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"
#include "swiglu.hpp"

namespace mx {

using v2::v16f;

struct KMapPlain {
  int64_t K;   // bytes
  __device__ __forceinline__ void operator()(int s, uint32_t& kc, int& kv) const {
    kc = uint32_t(int64_t(s) * v2::BK);
    const int64_t rem = K - int64_t(kc);
    kv = rem < v2::BK ? int(rem) : v2::BK;
  }
};

// ---------------------------------------------------------------------------
template <int BM, int BN, int FG, bool BIAS, bool GENERIC>
__global__ void __launch_bounds__(v2::kThreads) phase1_kernel(Phase1Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * v2::BK];
  constexpr int FM = BM / 64, FN = BN / 64;
  const int per_blk = p.tiles_m * p.tiles_n;
  const int id = v2::xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per_blk;
  int tm, tn;
  v2::grouped_tile<8>(id - b * per_blk, p.tiles_m, p.tiles_n, tm, tn);
  if (!p.flag[b]) return;
  const int64_t e = p.b2e[b];
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // m: i, n: slot within block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t P = p.N * p.B;
  const int64_t sbase = int64_t(b) * p.B;

  // A: dequantised W_down[e] rows i; B: dequantised dY rows gathered by token
  v2::Operand<BM, FM> A;
  v2::Operand<BN, FN> B;
  v2::setup_rows(A, reinterpret_cast<const uint8_t*>(p.wd_deq + e * p.I * p.H), nullptr, m0, p.I, 2 * p.H, 0,
                 (wave >> 1) * (BM / 2));
  const int32_t* st = p.slot_tok + sbase;
  const int64_t B_ = p.B;
  v2::setup_gather(B, reinterpret_cast<const uint8_t*>(p.dy_deq), nullptr, p.T, 2 * p.H, 0, (wave & 1) * (BN / 2),
                   [&](int r) -> int64_t { const int64_t s = n0 + r; return s < B_ ? int64_t(st[s]) : -1; });
  v16f acc[FM][FN];
  v2::mainloop<BM, BN, v2::kBf16, 0, 0, GENERIC>(A, B, int((2 * p.H + v2::BK - 1) / v2::BK), KMapPlain{2 * p.H},
                                                  smem, acc);

  // ---- epilogue -------------------------------------------------------------
  const int h = lane >> 5;
  const int64_t twoI = 2 * p.I;
#pragma unroll
  for (int fj = 0; fj < FN; ++fj) {
    const int64_t s = n0 + v2::acc_col<BM, BN>(fj);           // this lane's slot
    const bool in_blk = s < p.B;
    const int64_t slot = sbase + (in_blk ? s : 0);
    const bool valid = in_blk && p.slot_tok[slot] >= 0;
    const float a = valid ? p.slot_aff[slot] : 0.f;
    float daff = 0.f;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      const int64_t i0 = m0 + (wave >> 1) * (BM / 2) + fi * 32;   // first row of the fragment
      if (i0 >= p.I) continue;                                     // uniform per wave
      float dg[16], du[16];
      uint32_t amg = 0, amu = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t i = i0 + 8 * (q >> 2) + 4 * h + (q & 3);
        float g = 0.f, u = 0.f;
        if (valid) {
          g = bf16_to_f32(p.ckpt[((int64_t(b) * 2 + 0) * p.I + i) * p.B + s]);
          u = bf16_to_f32(p.ckpt[((int64_t(b) * 2 + 1) * p.I + i) * p.B + s]);
        }
        const float ga = swiglu_gate_act(g);
        const float inter = bf16_to_f32(f32_to_bf16(ga * u));
        const float ds = acc[fi][fj][q];
        daff += ds * inter;
        const float dinter = a * ds;
        dg[q] = bf16_to_f32(f32_to_bf16(dinter * u * dsilu_f32(g)));
        du[q] = bf16_to_f32(f32_to_bf16(dinter * ga));
        amg = max(amg, abs_bits(dg[q]));
        amu = max(amu, abs_bits(du[q]));
      }
      // along I: the 32 rows of this fragment are this lane's 16 and lane^32's 16
      amg = max(amg, uint32_t(__shfl_xor(int(amg), 32, 64)));
      amu = max(amu, uint32_t(__shfl_xor(int(amu), 32, 64)));
      if (in_blk) {
        const int Xg = scale_exp<FG>(amg), Xu = scale_exp<FG>(amu);
        uint8_t* rg = p.dgu_row_codes + slot * twoI + i0 + 4 * h;
        uint8_t* ru = rg + p.I;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t wg = 0, wu = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            wg |= encode<FG>(__float_as_uint(dg[4 * k + c]), Xg) << (8 * c);
            wu |= encode<FG>(__float_as_uint(du[4 * k + c]), Xu) << (8 * c);
          }
          *reinterpret_cast<uint32_t*>(rg + 8 * k) = wg;
          *reinterpret_cast<uint32_t*>(ru + 8 * k) = wu;
        }
        if (h == 0) {
          p.dgu_row_scales[slot * (twoI / 32) + i0 / 32] = uint8_t(Xg + 127);
          p.dgu_row_scales[slot * (twoI / 32) + (p.I + i0) / 32] = uint8_t(Xu + 127);
        }
      }
      // along the slots: a group is the 32 columns of this fragment (lanes of one half)
      const int64_t p0 = sbase + n0 + (wave & 1) * (BN / 2) + fj * 32;   // first slot of the group
      if (n0 + (wave & 1) * (BN / 2) + fj * 32 < p.B) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t i = i0 + 8 * (q >> 2) + 4 * h + (q & 3);
          uint32_t mg = abs_bits(dg[q]), mu = abs_bits(du[q]);
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) {
            mg = max(mg, uint32_t(__shfl_xor(int(mg), o, 64)));
            mu = max(mu, uint32_t(__shfl_xor(int(mu), o, 64)));
          }
          const int Xg = scale_exp<FG>(mg), Xu = scale_exp<FG>(mu);
          p.dgu_tok_codes[i * P + p0 + (lane & 31)] = uint8_t(encode<FG>(__float_as_uint(dg[q]), Xg));
          p.dgu_tok_codes[(p.I + i) * P + p0 + (lane & 31)] = uint8_t(encode<FG>(__float_as_uint(du[q]), Xu));
          if ((lane & 31) == 0) {
            p.dgu_tok_scales[i * (P / 32) + p0 / 32] = uint8_t(Xg + 127);
            p.dgu_tok_scales[(p.I + i) * (P / 32) + p0 / 32] = uint8_t(Xu + 127);
          }
          if (BIAS) {
            float sg = dg[q], su = du[q];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
              sg += __shfl_xor(sg, o, 64);
              su += __shfl_xor(su, o, 64);
            }
            if ((lane & 31) == 0) {
              atomicAdd(p.db1_acc + (e * 2 + 0) * p.I + i, sg);
              atomicAdd(p.db1_acc + (e * 2 + 1) * p.I + i, su);
            }
          }
        }
      }
    }
    // d(a): combine the two lane halves (same slot), then one atomic per slot
    daff += __shfl_xor(daff, 32, 64);
    if (valid && h == 0) atomicAdd(p.daff_slot + slot, daff);
  }
}

// ---------------------------------------------------------------------------
template <int BM, int BN, int FG, int FW, bool GENERIC>
__global__ void __launch_bounds__(v2::kThreads) phase3_kernel(Phase3Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * v2::BK];
  constexpr int FM = BM / 64, FN = BN / 64;
  const int per_blk = p.tiles_m * p.tiles_n;
  const int id = v2::xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per_blk;
  int tm, tn;
  v2::grouped_tile<8>(id - b * per_blk, p.tiles_m, p.tiles_n, tm, tn);
  if (!p.flag[b]) return;
  const int64_t e = p.b2e[b];
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // m: slot within block, n: h
  const int wave = threadIdx.x >> 6;
  const int64_t sbase = int64_t(b) * p.B;
  const int64_t twoI = 2 * p.I;

  // A: the block's rows of dGU quantised along I; B: W_gate_up[e] viewed [H][2I]
  v2::Operand<BM, FM> A;
  v2::Operand<BN, FN> B;
  v2::setup_rows(A, p.dgu_row_codes + sbase * twoI, p.dgu_row_scales + sbase * (twoI / 32), m0, p.B, twoI,
                 twoI / 32, (wave >> 1) * (BM / 2));
  v2::setup_rows(B, p.wgu_codes + e * p.H * twoI, p.wgu_scales + e * p.H * (twoI / 32), n0, p.H, twoI, twoI / 32,
                 (wave & 1) * (BN / 2));
  v16f acc[FM][FN];
  v2::mainloop<BM, BN, v2::kFp8, FG, FW, GENERIC>(A, B, int((twoI + v2::BK - 1) / v2::BK), KMapPlain{twoI}, smem,
                                                   acc);

#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t s = m0 + v2::acc_row<BM, BN>(fi, q);
      const int64_t tok = s < p.B ? p.slot_tok[sbase + s] : -1;
      if (tok < 0) continue;
      float* dst = p.dx_acc + tok * p.H;
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int64_t hh = n0 + v2::acc_col<BM, BN>(fj);
        if (hh < p.H) atomicAdd(dst + hh, acc[fi][fj][q]);
      }
    }
}

// ---------------------------------------------------------------------------
template <int BM, int BN, bool G>
static hipError_t phase1_launch(Phase1Args p, int fg, bool bias, hipStream_t st) {
  p.tiles_m = int((p.I + BM - 1) / BM);
  p.tiles_n = int((p.B + BN - 1) / BN);
  const unsigned blocks = unsigned(int64_t(p.tiles_m) * p.tiles_n * p.N);
  if (fg == 0) {
    if (bias) phase1_kernel<BM, BN, 0, true, G><<<blocks, v2::kThreads, 0, st>>>(p);
    else phase1_kernel<BM, BN, 0, false, G><<<blocks, v2::kThreads, 0, st>>>(p);
  } else {
    if (bias) phase1_kernel<BM, BN, 1, true, G><<<blocks, v2::kThreads, 0, st>>>(p);
    else phase1_kernel<BM, BN, 1, false, G><<<blocks, v2::kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

// Tile shape: 256 along a dimension when it is at least 256, else 128.
hipError_t launch_phase1(const Phase1Args& p, int fg, bool bias, hipStream_t st) {
  const bool g = (2 * p.H) % v2::BK != 0;      // a ragged last K stage
  if (p.I >= 256 && p.B >= 256)
    return g ? phase1_launch<256, 256, true>(p, fg, bias, st) : phase1_launch<256, 256, false>(p, fg, bias, st);
  if (p.I >= 256)
    return g ? phase1_launch<256, 128, true>(p, fg, bias, st) : phase1_launch<256, 128, false>(p, fg, bias, st);
  return g ? phase1_launch<128, 128, true>(p, fg, bias, st) : phase1_launch<128, 128, false>(p, fg, bias, st);
}

template <int BM, int BN, bool G>
static hipError_t phase3_launch(Phase3Args p, int fg, int fw, hipStream_t st) {
  p.tiles_m = int((p.B + BM - 1) / BM);
  p.tiles_n = int((p.H + BN - 1) / BN);
  const unsigned blocks = unsigned(int64_t(p.tiles_m) * p.tiles_n * p.N);
  if (fg == 0 && fw == 0) phase3_kernel<BM, BN, 0, 0, G><<<blocks, v2::kThreads, 0, st>>>(p);
  else if (fg == 0) phase3_kernel<BM, BN, 0, 1, G><<<blocks, v2::kThreads, 0, st>>>(p);
  else if (fw == 0) phase3_kernel<BM, BN, 1, 0, G><<<blocks, v2::kThreads, 0, st>>>(p);
  else phase3_kernel<BM, BN, 1, 1, G><<<blocks, v2::kThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_phase3(const Phase3Args& p, int fg, int fw, hipStream_t st) {
  const bool g = (2 * p.I) % v2::BK != 0;      // unaligned scale rows / ragged last K stage
  if (p.B >= 256 && p.H >= 256)
    return g ? phase3_launch<256, 256, true>(p, fg, fw, st) : phase3_launch<256, 256, false>(p, fg, fw, st);
  return g ? phase3_launch<128, 256, true>(p, fg, fw, st) : phase3_launch<128, 256, false>(p, fg, fw, st);
}

}  // namespace mx
