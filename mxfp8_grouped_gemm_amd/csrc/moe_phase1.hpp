// moe_phase1.hpp -- Phase 1 of the MoE backward with its fused SwiGLU-backward
// epilogue (P1, "Blockwise MM Backward MXFP8 Kernel API Reference": Phase 1
// and the checkpoint parameters; P3, sonic-moe functional/backward.py:
// _down_projection_backward_act).  The kernel template and its launcher; the
// tile shapes are instantiated in moe_phase1_*.hip so they compile in parallel.
//
// Per block b of expert e (tile rows = intermediate index i, tile columns =
// block slot p, contraction over H; the operands' exact MX values reduced with
// bf16 MFMAs, whose fp32 accumulation is exact enough that requantising the
// result below makes the same rounding decisions as an exact sum would):
//   dS[i][p]   = sum_h deq(W_down[e])[i][h] * deq(dY[tok_p])[h]   (dY rows are
//                quantised along H once and gathered here by token id)
//   epilogue:  ga = bf16(silu(g)), inter = bf16(ga*u)   (g,u from the checkpoint)
//              d(a)_p += sum_i dS*inter                  (fp32 atomics per slot)
//              dInter = a_p * dS
//              dGate = bf16(dInter*u*silu'(g)), dUp = bf16(dInter*ga)
//              -> quantised along I (Phase-3 A operand, [P][2I])
//              -> quantised along the slots (Phase-2 B operand, [2I][P])
//              -> db1 partial sums (with a bias)
#pragma once
#include "gemm_v2.hpp"
#include "gemm_v3.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"
#include "swiglu.hpp"

namespace mx {

using v2::v16f;
using v2::KMapPlain;

// ---------------------------------------------------------------------------
// Phase 1.  Epilogue data flow per wave (wave tile (BM/2) i-rows x (BN/2) slots):
//   for each 32-row fragment row fi:
//     for each fragment fj: SwiGLU backward on the 16 values a lane holds (one
//       slot, 16 of the 32 rows; lane^32 holds the other 16), the I-axis MX
//       groups (one xor-32 exchange for the amax), stores of dGU quantised
//       along I, and staging of dG|dU and the intermediate in LDS;
//     then each lane takes one staged row i and 32-slot groups of it, so the
//       slot-axis MX groups (dGU and the intermediate operand of Phase 4) are
//       reduced and encoded in registers and stored as 32-byte runs.
// The LDS of the main loop is reused for staging after a barrier.
template <int BM, int BN, int FG, int FW, bool ON_I, bool GENERIC>
__global__ void __launch_bounds__(v2::kThreads) phase1_kernel(Phase1Args p) {
  // GENERIC: H not a multiple of 128 (v2 loop on the bf16 values); otherwise the
  // ring (v3 loop) on the codes: fp8 in memory and LDS, exact bf16 on the MFMA
  constexpr int SMEM = GENERIC ? 2 * (BM + BN) * v2::BK : v3::smem_bytes(BM, BN);
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int WN = BN / 2;            // slots per wave
  constexpr int GS = WN * 4 + 16;       // staged row of dG | dU << 16 words (padding spreads rows over banks)
  constexpr int IS = WN * 2 + 16;       // staged row of intermediate bf16 values
  static_assert(4 * 32 * (GS + IS) <= SMEM, "per-wave staging must fit in the main-loop LDS");
  const int per_blk = p.tiles_m * p.tiles_n;
  const int id = v2::xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per_blk;
  int tm, tn;
  v2::grouped_tile<8>(id - b * per_blk, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // m: i, n: slot within block
  const int64_t P = p.N * p.B;
  const int64_t sbase = int64_t(b) * p.B;
  if (!p.flag[b]) {
    // a block without tokens: its intermediate operand is all zeros (codes 0, scale
    // byte 0; scales pair-major [P/128][I][4])
    for (int k = threadIdx.x; k < BM * (BN / 16); k += v2::kThreads) {
      const int64_t i = m0 + k / (BN / 16);
      if (i < p.I)
        *reinterpret_cast<uint4*>(p.inter_tok_codes + i * P + sbase + n0 + (k % (BN / 16)) * 16) = uint4{0, 0, 0, 0};
    }
    for (int k = threadIdx.x; k < BM * (BN / 128); k += v2::kThreads) {
      const int64_t i = m0 + k / (BN / 128);
      if (i < p.I)
        *reinterpret_cast<uint32_t*>(p.inter_tok_scales + (((sbase + n0) / 128 + k % (BN / 128)) * p.I + i) * 4) = 0u;
    }
    return;
  }
  const int64_t e = p.b2e[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  const int32_t* st = p.slot_tok + sbase;
  const int64_t B_ = p.B;
  auto tok_of = [&](int r) -> int64_t { const int64_t s = n0 + r; return s < B_ ? int64_t(st[s]) : -1; };
  v16f acc[FM][FN];
  if constexpr (GENERIC) {
    // A: dequantised W_down[e] rows i; B: dequantised dY rows gathered by token
    const uint8_t* wd = reinterpret_cast<const uint8_t*>(p.wd_deq + e * p.I * p.H);
    const uint8_t* dyd = reinterpret_cast<const uint8_t*>(p.dy_deq);
    v2::Operand<BM, FM> A;
    v2::Operand<BN, FN> B;
    v2::setup_rows(A, wd, nullptr, m0, p.I, 2 * p.H, 0, (wave >> 1) * (BM / 2));
    v2::setup_gather(B, dyd, nullptr, p.T, 2 * p.H, 0, (wave & 1) * (BN / 2), tok_of);
    v2::mainloop<BM, BN, v2::kBf16, 0, 0, true>(A, B, int((2 * p.H + v2::BK - 1) / v2::BK), KMapPlain{2 * p.H},
                                                 smem, acc);
  } else {
    // A: W_down[e] codes rows i; B: Q_H(dY) codes rows gathered by token
    v3::Op<BM> A;
    v3::Op<BN> B;
    v3::setup_rows(A, p.wd_codes + e * p.I * p.H, m0, p.I, p.H);
    v3::setup_gather(B, p.dy_codes, p.T, p.H, tok_of);
    v3::ScaleDma<BM, BN> sd;
    const int64_t I_ = p.I;
    v3::setup_scales_map(
        sd, p.wd_scales + e * p.I * (p.H / 32), p.I, p.I * (p.H / 32),
        [&](int r) -> int64_t { return m0 + r < I_ ? m0 + r : -1; }, p.dy_scales, p.T, p.T * (p.H / 32), tok_of);
    v3::mainloop<BM, BN, v3::kFp8Bf16, FW, FG>(A, B, &sd, int(p.H / v3::SK), v3::KMapPlain{}, smem, acc);
  }

  // ---- epilogue -------------------------------------------------------------
  __syncthreads();   // every wave has read the last stage: the LDS is free for staging
  const int h = lane >> 5, r = lane & 31;
  const int wrow = (wave >> 1) * (BM / 2), wcol = (wave & 1) * (BN / 2);
  uint8_t* stg_gu = smem + wave * 32 * (GS + IS);
  uint8_t* stg_in = stg_gu + 32 * GS;
  const int64_t twoI = 2 * p.I;
  // the block's checkpoint [2][I][B] bf16 through a buffer: padding slots read as zeros
  [[maybe_unused]] const v2::Buf ck = v2::make_rsrc(p.ckpt + int64_t(b) * 2 * p.I * p.B, uint32_t(4 * p.I * p.B));
  [[maybe_unused]] const uint32_t up_plane = uint32_t(2 * p.I * p.B);
  float aff[FN], daff[FN];
  uint32_t ckoff[FN];
  v2::static_for<FN>([&](auto FJ) {
    constexpr int fj = FJ;
    const int64_t s = n0 + wcol + fj * 32 + r;
    const bool ok = st[s] >= 0;
    aff[fj] = ok ? p.slot_aff[sbase + s] : 0.f;
    daff[fj] = 0.f;
    ckoff[fj] = ok ? uint32_t((4 * h * p.B + s) * 2) : v2::kOOB;   // row 4h of a fragment, this slot
  });

  v2::static_for<FM>([&](auto FI) {
    constexpr int fi = FI;
    const int64_t i0 = m0 + wrow + fi * 32;   // first row of the fragment row; I % 32 == 0
    if (i0 < p.I) {                           // wave-uniform
      v2::static_for<FN>([&](auto FJ) {
        constexpr int fj = FJ;
        uint16_t gb[16], ub[16];
#if defined(__HIP_DEVICE_COMPILE__)
        const auto rs = MX_RSRC(ck);
        v2::static_for<16>([&](auto Q) {
          constexpr int q = Q;
          const uint32_t so =
              __builtin_amdgcn_readfirstlane(uint32_t((i0 + 8 * (q >> 2) + (q & 3)) * p.B * 2));
          gb[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, ckoff[fj], so, 0);
          ub[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, ckoff[fj], so + up_plane, 0);
        });
#endif
        uint32_t gu[16];        // bf16(dGate) | bf16(dUp) << 16
        uint16_t it[16];        // bf16 intermediate operand (times a with the affinity on I)
        float amg = 0.f, amu = 0.f;
        v2::static_for<16>([&](auto Q) {
          constexpr int q = Q;
          const float g = bf16_to_f32(gb[q]), u = bf16_to_f32(ub[q]);
          const float sg = sigmoid_fast(g);
          const float ga = bf16_round(g * sg);           // silu(g)
          const float in = bf16_round(ga * u);           // intermediate
          const float ds = acc[fi][fj][q];
          daff[fj] += ds * in;
          const float di = aff[fj] * ds;                 // d(intermediate)
          gu[q] = bf16x2_rne(di * u * dsilu_from(g, sg), di * ga);
          it[q] = ON_I ? bf16_rne(aff[fj] * in) : uint16_t(__float_as_uint(in) >> 16);
          amg = fmaxf(amg, fabsf(lo_bf16(gu[q])));
          amu = fmaxf(amu, fabsf(hi_bf16(gu[q])));
        });
        // I-axis groups: the fragment's 32 rows are this lane's 16 and lane^32's 16
        amg = fmaxf(amg, __shfl_xor(amg, 32, 64));
        amu = fmaxf(amu, __shfl_xor(amu, 32, 64));
        const int Xg = scale_exp<FG>(__float_as_uint(amg)), Xu = scale_exp<FG>(__float_as_uint(amu));
        const float ig = inv_scale(Xg), iu = inv_scale(Xu);
        const int64_t slot = sbase + n0 + wcol + fj * 32 + r;
        uint8_t* rg = p.dgu_row_codes + slot * twoI + i0 + 4 * h;
        uint8_t* ru = rg + p.I;
        v2::static_for<4>([&](auto K) {
          constexpr int k = K;
          *reinterpret_cast<uint32_t*>(rg + 8 * k) = encode4<FG>(lo_bf16(gu[4 * k]), lo_bf16(gu[4 * k + 1]),
                                                                 lo_bf16(gu[4 * k + 2]), lo_bf16(gu[4 * k + 3]), ig);
          *reinterpret_cast<uint32_t*>(ru + 8 * k) = encode4<FG>(hi_bf16(gu[4 * k]), hi_bf16(gu[4 * k + 1]),
                                                                 hi_bf16(gu[4 * k + 2]), hi_bf16(gu[4 * k + 3]), iu);
        });
        if (h == 0) {
          const int64_t gg = i0 / 32, gu_ = (p.I + i0) / 32;
          if (p.dgu_row_pairs) {   // pair-major [2I/128][P][4]
            p.dgu_row_scales[((gg >> 2) * P + slot) * 4 + (gg & 3)] = uint8_t(Xg + 127);
            p.dgu_row_scales[((gu_ >> 2) * P + slot) * 4 + (gu_ & 3)] = uint8_t(Xu + 127);
          } else {                 // row-major [P][2I/32]
            p.dgu_row_scales[slot * (twoI / 32) + gg] = uint8_t(Xg + 127);
            p.dgu_row_scales[slot * (twoI / 32) + gu_] = uint8_t(Xu + 127);
          }
        }
        // staging for the slot-axis groups
        v2::static_for<16>([&](auto Q) {
          constexpr int q = Q;
          const int row = 8 * (q >> 2) + 4 * h + (q & 3), col = fj * 32 + r;
          *reinterpret_cast<uint32_t*>(stg_gu + row * GS + col * 4) = gu[q];
          *reinterpret_cast<uint16_t*>(stg_in + row * IS + col * 2) = it[q];
        });
      });
      // the staging writes of this wave are visible to its own later reads (LDS is in order per wave)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // slot-axis groups: lane takes row r of the fragment row, groups h, h+2, ...
      const int64_t i = i0 + r;
      v2::static_for<FN / 2>([&](auto C) {
        const int c = h + 2 * int(C);
        const int64_t p0 = sbase + n0 + wcol + c * 32;
        uint4 w[8];
        v2::static_for<8>([&](auto J) {
          w[J] = *reinterpret_cast<const uint4*>(stg_gu + r * GS + c * 128 + 16 * int(J));
        });
        uint32_t mg = 0, mu = 0;
        float sg = 0.f, su = 0.f;
        v2::static_for<8>([&](auto J) {
          const uint32_t x[4] = {w[J].x, w[J].y, w[J].z, w[J].w};
          v2::static_for<4>([&](auto T) {
            mg = max(mg, (x[T] << 16) & 0x7fffffffu);
            mu = max(mu, x[T] & 0x7fff0000u);
            if (p.has_bias) {
              sg += __uint_as_float(x[T] << 16);
              su += __uint_as_float(x[T] & 0xffff0000u);
            }
          });
        });
        const int Xg = scale_exp<FG>(mg), Xu = scale_exp<FG>(mu);
        const float ig = inv_scale(Xg), iu = inv_scale(Xu);
        uint32_t cg[8], cu[8];
        v2::static_for<8>([&](auto J) {
          const uint32_t x[4] = {w[J].x, w[J].y, w[J].z, w[J].w};
          cg[J] = encode4<FG>(__uint_as_float(x[0] << 16), __uint_as_float(x[1] << 16), __uint_as_float(x[2] << 16),
                              __uint_as_float(x[3] << 16), ig);
          cu[J] = encode4<FG>(__uint_as_float(x[0] & 0xffff0000u), __uint_as_float(x[1] & 0xffff0000u),
                              __uint_as_float(x[2] & 0xffff0000u), __uint_as_float(x[3] & 0xffff0000u), iu);
        });
        uint4* og = reinterpret_cast<uint4*>(p.dgu_tok_codes + i * P + p0);
        uint4* ou = reinterpret_cast<uint4*>(p.dgu_tok_codes + (p.I + i) * P + p0);
        og[0] = uint4{cg[0], cg[1], cg[2], cg[3]};
        og[1] = uint4{cg[4], cg[5], cg[6], cg[7]};
        ou[0] = uint4{cu[0], cu[1], cu[2], cu[3]};
        ou[1] = uint4{cu[4], cu[5], cu[6], cu[7]};
        const int64_t g32 = p0 / 32;   // pair-major [P/128][2I][4]
        p.dgu_tok_scales[((g32 >> 2) * twoI + i) * 4 + (g32 & 3)] = uint8_t(Xg + 127);
        p.dgu_tok_scales[((g32 >> 2) * twoI + p.I + i) * 4 + (g32 & 3)] = uint8_t(Xu + 127);
        if (p.has_bias) {
          atomicAdd(p.db1_acc + (e * 2 + 0) * p.I + i, sg);
          atomicAdd(p.db1_acc + (e * 2 + 1) * p.I + i, su);
        }
        // the intermediate operand (activation format)
        uint4 v[4];
        v2::static_for<4>([&](auto J) {
          v[J] = *reinterpret_cast<const uint4*>(stg_in + r * IS + c * 64 + 16 * int(J));
        });
        uint32_t mi = 0;
        v2::static_for<4>([&](auto J) {
          const uint32_t x[4] = {v[J].x, v[J].y, v[J].z, v[J].w};
          v2::static_for<4>([&](auto T) {
            mi = max(mi, (x[T] << 16) & 0x7fffffffu);
            mi = max(mi, x[T] & 0x7fff0000u);
          });
        });
        const bool e5 = p.fmt_act == kE5M2;   // wave-uniform
        const int Xi = e5 ? scale_exp<kE5M2>(mi) : scale_exp<kE4M3>(mi);
        const float ii = inv_scale(Xi);
        uint32_t ci[8];
        v2::static_for<4>([&](auto J) {
          const uint32_t x[4] = {v[J].x, v[J].y, v[J].z, v[J].w};
          if (e5) {
            ci[2 * J] = encode4<kE5M2>(lo_bf16(x[0]), hi_bf16(x[0]), lo_bf16(x[1]), hi_bf16(x[1]), ii);
            ci[2 * J + 1] = encode4<kE5M2>(lo_bf16(x[2]), hi_bf16(x[2]), lo_bf16(x[3]), hi_bf16(x[3]), ii);
          } else {
            ci[2 * J] = encode4<kE4M3>(lo_bf16(x[0]), hi_bf16(x[0]), lo_bf16(x[1]), hi_bf16(x[1]), ii);
            ci[2 * J + 1] = encode4<kE4M3>(lo_bf16(x[2]), hi_bf16(x[2]), lo_bf16(x[3]), hi_bf16(x[3]), ii);
          }
        });
        uint4* oi = reinterpret_cast<uint4*>(p.inter_tok_codes + i * P + p0);
        oi[0] = uint4{ci[0], ci[1], ci[2], ci[3]};
        oi[1] = uint4{ci[4], ci[5], ci[6], ci[7]};
        p.inter_tok_scales[((g32 >> 2) * p.I + i) * 4 + (g32 & 3)] = uint8_t(Xi + 127);   // [P/128][I][4]
      });
      // the next fragment row overwrites the staging only after these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  });
  // d(a): the two lane halves hold the same slot; one atomic per slot and wave
  v2::static_for<FN>([&](auto FJ) {
    constexpr int fj = FJ;
    const float d = daff[fj] + __shfl_xor(daff[fj], 32, 64);
    const int64_t s = n0 + wcol + fj * 32 + r;
    if (h == 0 && st[s] >= 0) atomicAdd(p.daff_slot + sbase + s, d);
  });
}

// ---------------------------------------------------------------------------
template <int BM, int BN, bool G, int FG, int FW>
inline void phase1_go(const Phase1Args& p, unsigned blocks, hipStream_t st) {
  if (p.affinity_on_i) phase1_kernel<BM, BN, FG, FW, true, G><<<blocks, v2::kThreads, 0, st>>>(p);
  else phase1_kernel<BM, BN, FG, FW, false, G><<<blocks, v2::kThreads, 0, st>>>(p);
}

template <int BM, int BN, bool G>
hipError_t phase1_launch(Phase1Args p, int fg, int fw, hipStream_t st) {
  p.tiles_m = int((p.I + BM - 1) / BM);
  p.tiles_n = int((p.B + BN - 1) / BN);
  const int64_t blocks = int64_t(p.tiles_m) * p.tiles_n * p.N;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const unsigned grid = unsigned(blocks);
  if (G) {   // the bf16 values carry no format
    if (fg == kE4M3) phase1_go<BM, BN, G, kE4M3, kE4M3>(p, grid, st);
    else phase1_go<BM, BN, G, kE5M2, kE4M3>(p, grid, st);
  } else if (fg == kE4M3) {
    if (fw == kE4M3) phase1_go<BM, BN, G, kE4M3, kE4M3>(p, grid, st);
    else phase1_go<BM, BN, G, kE4M3, kE5M2>(p, grid, st);
  } else {
    if (fw == kE4M3) phase1_go<BM, BN, G, kE5M2, kE4M3>(p, grid, st);
    else phase1_go<BM, BN, G, kE5M2, kE5M2>(p, grid, st);
  }
  return hipGetLastError();
}

}  // namespace mx
