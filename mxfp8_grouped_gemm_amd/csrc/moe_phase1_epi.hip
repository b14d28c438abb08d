// moe_phase1_epi.hip -- the SwiGLU (or GeGLU) backward after Phase 1's product (P1,
// "Blockwise MM Backward MXFP8 Kernel API Reference": Phase 1's epilogue and
// the checkpoint parameters; P3, sonic-moe functional/backward.py:
// _down_projection_backward_act, the gated-activation backward).
//
// Per slot p of block b (token t, affinity a_p; padding slots contribute zeros)
// and intermediate index i, from dS = Phase 1's product and the checkpoint g, u:
//   ga = bf16(silu(g)) (GeGLU: bf16(gelu(g))), inter = bf16(ga * u)
//   d(a)_p  = sum_i dS * inter                  (a partial per 32 rows i, summed
//                                                at the end in order)
//   dInter = a_p * dS
//   dGate = bf16(dInter * u * silu'(g)) (GeGLU: gelu'(g)), dUp = bf16(dInter * ga)
//   -> quantised along I        (Phase-3 A operand, dgu_row [P][2I])
//   -> quantised along the slots (Phase-2 B operand, dgu_tok [2I][P])
//   -> db1 partial sums along the slots (with a bias)
//   the intermediate operand of Phase 4 (times a_p with the affinity on I),
//   quantised along the slots (inter_tok [I][P]); blocks without tokens get zeros.
//
// HBM-bound: a workgroup takes a tile of TI rows i x TS slots of one block
// (TS = min(B, 256), TI * TS = 8192).  Pass 1, one thread per (slot, 32 rows):
// coalesced loads of dS and the checkpoint, the element-wise math, the I-axis
// groups in registers and their 32-byte code runs, d(a) partials; dG|dU and the
// intermediate are staged in LDS.  Pass 2, one thread per (row, 32-slot group):
// the slot-axis groups from LDS, stored as 32-byte runs.
#include "kernels.hpp"
#include "gemm_v2.hpp"
#include "mx_device.hpp"
#include "swiglu.hpp"

namespace mx {

namespace {
constexpr int kEpiThreads = 256;
constexpr int kEpiElems = 8192;   // TI * TS
}  // namespace

// The element-wise SwiGLU backward of one (slot, i): from dS = d, the
// checkpoint's g and u and the affinity a, adds this element's share of d(a)
// and returns bf16(dGate) | bf16(dUp) << 16 and the bf16 intermediate operand.
// A supplied checkpoint value (HAS_*) replaces the recomputed one; the values
// are rounded at the same points either way, so consistent checkpoints give
// the same bits.
// GEGLU: the gate activation is gelu (g * Phi(g)) instead of silu.
template <bool ON_I, bool GEGLU>
__device__ __forceinline__ uint32_t swiglu_bwd(float d, float g, float u, float a, bool has_ga, float ga_in,
                                               bool has_in, float in_in, bool has_sc, uint16_t sc_in, float& daff,
                                               uint16_t& it) {
  if constexpr (GEGLU) {
    const float cdf = normal_cdf(g);
    const float ga = has_ga ? ga_in : bf16_round(g * cdf);   // gelu(g)
    const float in = has_in ? in_in : bf16_round(ga * u);    // intermediate
    daff += d * in;
    const float di = a * d;                                  // d(intermediate)
    it = ON_I ? (has_sc ? sc_in : bf16_rne(a * in)) : uint16_t(__float_as_uint(in) >> 16);
    return bf16x2_rne(di * u * dgelu_from(g, cdf), di * ga);
  } else {
    const float sg = sigmoid_fast(g);
    const float ga = has_ga ? ga_in : bf16_round(g * sg);   // silu(g)
    const float in = has_in ? in_in : bf16_round(ga * u);   // intermediate
    daff += d * in;
    const float di = a * d;                                 // d(intermediate)
    it = ON_I ? (has_sc ? sc_in : bf16_rne(a * in)) : uint16_t(__float_as_uint(in) >> 16);
    return bf16x2_rne(di * u * dsilu_from(g, sg), di * ga);
  }
}

// CK: the caller supplied at least one of the [N][I][B] checkpoints (silu(gate),
// the intermediate, the scaled intermediate); pass 1 then runs its 32 rows in
// two halves so that the extra loads fit in registers.
template <int FG, bool ON_I, int TS, bool CK, bool GEGLU>
__global__ void __launch_bounds__(kEpiThreads) phase1_epi_kernel(Phase1Args p) {
  constexpr int TI = kEpiElems / TS;         // rows of the tile
  constexpr int NG = TS / 32;                // 32-slot groups of a row
  // Staging: row r, slot s at r * GSW + (s / 32) * 33 + s % 32 (dG|dU words) and
  // r * ISH + (s / 32) * 34 + s % 32 (intermediate values).  Pass 2's lanes read
  // rows r..r+7, groups c = 0..7 at one offset: word 8r + 33c (+ k) mod 64 is a
  // different bank for each lane, and pass 1's lanes write consecutive words.
  constexpr int GSW = 33 * NG, ISH = 34 * NG;
  __shared__ uint32_t stg_gu[TI * GSW];
  __shared__ uint16_t stg_in[TI * ISH];
  // Tile order: the 128 / TI row tiles that share a slot's 128-byte run of
  // dgu_row codes and its scale words are consecutive, and consecutive tiles
  // run on one XCD, so those lines fill up in one L2 instead of reaching HBM
  // in pieces from several.
  constexpr int GI = 128 / TI;
  const int tiles_i = int((p.I + TI - 1) / TI), tiles_s = int(p.B / TS);
  const int per_b = tiles_i * tiles_s;
  const int id = v2::xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per_b;
  int tile_i, tile_s;
  v2::grouped_tile<GI>(id - b * per_b, tiles_i, tiles_s, tile_i, tile_s);
  const int64_t ti0 = int64_t(tile_i) * TI, s0 = int64_t(tile_s) * TS;
  const int64_t P = p.N * p.B, twoI = 2 * p.I;
  const int64_t sbase = int64_t(b) * p.B;
  const int t = threadIdx.x;

  if (!p.flag[b]) {
    // a block without tokens: its intermediate operand is all zeros (codes 0,
    // scale byte 0; scales pair-major [P/128][I][4])
    for (int k = t; k < TI * (TS / 16); k += kEpiThreads) {
      const int64_t i = ti0 + k / (TS / 16);
      if (i < p.I)
        *reinterpret_cast<uint4*>(p.inter_tok_codes + i * P + sbase + s0 + (k % (TS / 16)) * 16) = uint4{0, 0, 0, 0};
    }
    for (int k = t; k < TI * (TS / 128); k += kEpiThreads) {
      const int64_t i = ti0 + k / (TS / 128);
      if (i < p.I)
        *reinterpret_cast<uint32_t*>(p.inter_tok_scales + (((sbase + s0) / 128 + k % (TS / 128)) * p.I + i) * 4) = 0u;
    }
    return;
  }
  const int64_t e = p.b2e[b];

  // ---- pass 1: thread = slot s (of the tile) x 32 rows r0 .. r0 + 31 --------------
  {
    const int sl = t % TS, r0 = 32 * (t / TS);
    const int64_t slot = sbase + s0 + sl;
    const int64_t i0 = ti0 + r0;
    const bool ok = p.slot_tok[slot] >= 0;
    const float a = ok ? p.slot_aff[slot] : 0.f;
    if (i0 < p.I) {   // I % 32 == 0: all 32 rows or none
      // Buffer loads: row offsets are wave-uniform (scalar), the slot offset is
      // this lane's; padding slots load through an offset past the buffer, which
      // reads zeros, so no load is conditional (each would be a branch with its
      // own wait, serialising the 96 loads a thread keeps in flight).
      uint32_t gu[32];   // bf16(dGate) | bf16(dUp) << 16
      uint16_t it[32];   // bf16 intermediate operand
      float daff = 0.f, amg = 0.f, amu = 0.f;
#if defined(__HIP_DEVICE_COMPILE__)
      // a tile past the block's extent is all padding (dS unwritten there): its
      // descriptors have no records, so every load reads zero without memory traffic
      const uint32_t live = s0 < p.flag[b] ? 1u : 0u;
      const auto rd = MX_RSRC(v2::make_rsrc(p.ds + int64_t(b) * p.I * p.B, live * uint32_t(p.I * p.B * 4)));
      const auto rc = MX_RSRC(v2::make_rsrc(p.ckpt + int64_t(b) * 2 * p.I * p.B, live * uint32_t(p.I * p.B * 4)));
      // padding slots read dS and the checkpoint as zeros (their dS may be unwritten)
      const uint32_t vd = ok ? uint32_t((s0 + sl) * 4) : v2::kOOB, vc = ok ? uint32_t((s0 + sl) * 2) : v2::kOOB;
      if constexpr (!CK) {
        uint16_t gb[32], ub[32];
        float dv[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const uint32_t row = __builtin_amdgcn_readfirstlane(uint32_t((i0 + k) * p.B));
          dv[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, vd, row * 4, 0));
          gb[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, vc, row * 2, 0);
          ub[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, vc, (row + uint32_t(p.I * p.B)) * 2, 0);
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          gu[k] = swiglu_bwd<ON_I, GEGLU>(dv[k], bf16_to_f32(gb[k]), bf16_to_f32(ub[k]), a, false, 0.f, false, 0.f, false,
                                   0, daff, it[k]);
          amg = fmaxf(amg, fabsf(lo_bf16(gu[k])));
          amu = fmaxf(amu, fabsf(hi_bf16(gu[k])));
        }
      } else {
        // a checkpoint that was not supplied is read through a descriptor with
        // no records: zeros, no memory traffic, and the value is recomputed
        const bool has_ga = p.ga_ckpt != nullptr, has_in = p.in_ckpt != nullptr, has_sc = p.sc_ckpt != nullptr;
        const int64_t blk = int64_t(b) * p.I * p.B;
        const uint32_t ck_bytes = live * uint32_t(p.I * p.B * 2);
        const auto rga = MX_RSRC(v2::make_rsrc(has_ga ? p.ga_ckpt + blk : p.ckpt, has_ga ? ck_bytes : 0u));
        const auto rin = MX_RSRC(v2::make_rsrc(has_in ? p.in_ckpt + blk : p.ckpt, has_in ? ck_bytes : 0u));
        const auto rsc = MX_RSRC(v2::make_rsrc(has_sc ? p.sc_ckpt + blk : p.ckpt, has_sc ? ck_bytes : 0u));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint16_t gb[16], ub[16], gab[16], inb[16], scb[16];
          float dv[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const uint32_t row = __builtin_amdgcn_readfirstlane(uint32_t((i0 + 16 * hh + k) * p.B));
            dv[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, vd, row * 4, 0));
            gb[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, vc, row * 2, 0);
            ub[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, vc, (row + uint32_t(p.I * p.B)) * 2, 0);
            gab[k] = __builtin_amdgcn_raw_buffer_load_b16(rga, vc, row * 2, 0);
            inb[k] = __builtin_amdgcn_raw_buffer_load_b16(rin, vc, row * 2, 0);
            scb[k] = __builtin_amdgcn_raw_buffer_load_b16(rsc, vc, row * 2, 0);
          }
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const int kk = 16 * hh + k;
            gu[kk] = swiglu_bwd<ON_I, GEGLU>(dv[k], bf16_to_f32(gb[k]), bf16_to_f32(ub[k]), a, has_ga, bf16_to_f32(gab[k]),
                                      has_in, bf16_to_f32(inb[k]), has_sc, scb[k], daff, it[kk]);
            amg = fmaxf(amg, fabsf(lo_bf16(gu[kk])));
            amu = fmaxf(amu, fabsf(hi_bf16(gu[kk])));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#endif
      // I-axis groups: the thread's 32 rows are one group of dGate and one of dUp
      const int Xg = scale_exp<FG>(__float_as_uint(amg)), Xu = scale_exp<FG>(__float_as_uint(amu));
      const float ig = inv_scale(Xg), iu = inv_scale(Xu);
      uint32_t wg[8], wu[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        wg[k] = encode4<FG>(lo_bf16(gu[4 * k]), lo_bf16(gu[4 * k + 1]), lo_bf16(gu[4 * k + 2]), lo_bf16(gu[4 * k + 3]),
                            ig);
        wu[k] = encode4<FG>(hi_bf16(gu[4 * k]), hi_bf16(gu[4 * k + 1]), hi_bf16(gu[4 * k + 2]), hi_bf16(gu[4 * k + 3]),
                            iu);
      }
      uint4* rg = reinterpret_cast<uint4*>(p.dgu_row_codes + slot * twoI + i0);
      uint4* ru = reinterpret_cast<uint4*>(p.dgu_row_codes + slot * twoI + p.I + i0);
      rg[0] = uint4{wg[0], wg[1], wg[2], wg[3]};
      rg[1] = uint4{wg[4], wg[5], wg[6], wg[7]};
      ru[0] = uint4{wu[0], wu[1], wu[2], wu[3]};
      ru[1] = uint4{wu[4], wu[5], wu[6], wu[7]};
      const int64_t gg = i0 / 32, gu_ = (p.I + i0) / 32;
      if (p.dgu_row_pairs) {   // pair-major [2I/128][P][4]
        p.dgu_row_scales[((gg >> 2) * P + slot) * 4 + (gg & 3)] = uint8_t(Xg + 127);
        p.dgu_row_scales[((gu_ >> 2) * P + slot) * 4 + (gu_ & 3)] = uint8_t(Xu + 127);
      } else {                 // row-major [P][2I/32]
        p.dgu_row_scales[slot * (twoI / 32) + gg] = uint8_t(Xg + 127);
        p.dgu_row_scales[slot * (twoI / 32) + gu_] = uint8_t(Xu + 127);
      }
      p.daff_part[(i0 / 32) * P + slot] = daff;   // this 32-row group's share of d(a)
      // staging for the slot-axis groups: consecutive threads, consecutive slots
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        stg_gu[(r0 + k) * GSW + (sl >> 5) * 33 + (sl & 31)] = gu[k];
        stg_in[(r0 + k) * ISH + (sl >> 5) * 34 + (sl & 31)] = it[k];
      }
    }
  }
  __syncthreads();

  // ---- pass 2: thread = row r x 32-slot group c ---------------------------------------
  {
    const int r = t / NG, c = t % NG;
    const int64_t i = ti0 + r;
    if (i < p.I) {
      const int64_t p0 = sbase + s0 + 32 * c;
      const uint32_t* src = stg_gu + r * GSW + 33 * c;
      uint32_t mg = 0, mu = 0;
      float sg = 0.f, su = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint32_t x = src[k];
        mg = max(mg, (x << 16) & 0x7fffffffu);
        mu = max(mu, x & 0x7fff0000u);
        if (p.has_bias) {
          sg += __uint_as_float(x << 16);
          su += __uint_as_float(x & 0xffff0000u);
        }
      }
      const int Xg = scale_exp<FG>(mg), Xu = scale_exp<FG>(mu);
      const float ig = inv_scale(Xg), iu = inv_scale(Xu);
      uint32_t cg[8], cu[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t x0 = src[4 * k], x1 = src[4 * k + 1], x2 = src[4 * k + 2], x3 = src[4 * k + 3];
        cg[k] = encode4<FG>(lo_bf16(x0), lo_bf16(x1), lo_bf16(x2), lo_bf16(x3), ig);
        cu[k] = encode4<FG>(hi_bf16(x0), hi_bf16(x1), hi_bf16(x2), hi_bf16(x3), iu);
      }
      uint4* og = reinterpret_cast<uint4*>(p.dgu_tok_codes + i * P + p0);
      uint4* ou = reinterpret_cast<uint4*>(p.dgu_tok_codes + (p.I + i) * P + p0);
      og[0] = uint4{cg[0], cg[1], cg[2], cg[3]};
      og[1] = uint4{cg[4], cg[5], cg[6], cg[7]};
      ou[0] = uint4{cu[0], cu[1], cu[2], cu[3]};
      ou[1] = uint4{cu[4], cu[5], cu[6], cu[7]};
      const int64_t g32 = p0 / 32;   // pair-major [P/128][2I][4]
      p.dgu_tok_scales[((g32 >> 2) * twoI + i) * 4 + (g32 & 3)] = uint8_t(Xg + 127);
      p.dgu_tok_scales[((g32 >> 2) * twoI + p.I + i) * 4 + (g32 & 3)] = uint8_t(Xu + 127);
      if (p.has_bias) {   // the row's NG groups sit in consecutive lanes: one atomic per row
        for (int o = 1; o < NG; o <<= 1) {
          sg += __shfl_xor(sg, o, 64);
          su += __shfl_xor(su, o, 64);
        }
        if (c == 0) {
          atomicAdd(p.db1_acc + (e * 2 + 0) * p.I + i, sg);
          atomicAdd(p.db1_acc + (e * 2 + 1) * p.I + i, su);
        }
      }
      // the intermediate operand (activation format)
      const uint16_t* isrc = stg_in + r * ISH + 34 * c;
      uint32_t mi = 0;
#pragma unroll
      for (int k = 0; k < 32; ++k) mi = max(mi, (uint32_t(isrc[k]) << 16) & 0x7fffffffu);
      const bool e5 = p.fmt_act == kE5M2;   // uniform
      const int Xi = e5 ? scale_exp<kE5M2>(mi) : scale_exp<kE4M3>(mi);
      const float ii = inv_scale(Xi);
      uint32_t ci[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v0 = bf16_to_f32(isrc[4 * k]), v1 = bf16_to_f32(isrc[4 * k + 1]);
        const float v2 = bf16_to_f32(isrc[4 * k + 2]), v3 = bf16_to_f32(isrc[4 * k + 3]);
        ci[k] = e5 ? encode4<kE5M2>(v0, v1, v2, v3, ii) : encode4<kE4M3>(v0, v1, v2, v3, ii);
      }
      uint4* oi = reinterpret_cast<uint4*>(p.inter_tok_codes + i * P + p0);
      oi[0] = uint4{ci[0], ci[1], ci[2], ci[3]};
      oi[1] = uint4{ci[4], ci[5], ci[6], ci[7]};
      p.inter_tok_scales[((g32 >> 2) * p.I + i) * 4 + (g32 & 3)] = uint8_t(Xi + 127);   // [P/128][I][4]
    }
  }
}

template <int TS, bool CK, bool GEGLU>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  constexpr int TI = kEpiElems / TS;
  const int64_t grid = int64_t(p.N) * ((p.I + TI - 1) / TI) * (p.B / TS);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const bool on_i = p.affinity_on_i != 0;
  if (fg == kE4M3) {
    if (on_i) phase1_epi_kernel<kE4M3, true, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
    else phase1_epi_kernel<kE4M3, false, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
  } else {
    if (on_i) phase1_epi_kernel<kE5M2, true, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
    else phase1_epi_kernel<kE5M2, false, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}
template <int TS, bool GEGLU>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.ga_ckpt || p.in_ckpt || p.sc_ckpt) return epi_launch<TS, true, GEGLU>(p, fg, st);
  return epi_launch<TS, false, GEGLU>(p, fg, st);
}
template <int TS>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.geglu) return epi_launch<TS, true>(p, fg, st);
  return epi_launch<TS, false>(p, fg, st);
}

// Block size B: a power of two >= 128 (tiles of 256 slots, or of the whole block at 128).
hipError_t launch_phase1_epi(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.B % 256 == 0) return epi_launch<256>(p, fg, st);
  if (p.B == 128) return epi_launch<128>(p, fg, st);
  return hipErrorInvalidValue;
}

}  // namespace mx
