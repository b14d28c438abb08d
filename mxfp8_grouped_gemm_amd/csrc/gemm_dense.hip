// gemm_dense.hip -- MXFP8 NT GEMM with a bf16 store, for
//   * the dense backward (P2, "Matmul MXFP8 Backward Kernel API Reference"):
//       dX [M,K] = dY [M,N] . W^T [K,N]^T      (contraction over N)
//       dW [N,K] = dY^T [N,M] . X^T [K,M]^T    (contraction over M)
//   * the MoE weight gradients (P1 Phases 2 and 4), one group per expert,
//     whose contraction runs over the expert's blocks of token slots:
//       dW_gate_up[e] [H,2I] = X_tok [H,P] . dGU_tok [2I,P]^T
//       dW_down[e]    [I,H]  = inter_tok [I,P] . gy_tok [H,P]^T
//     where the K columns of expert e are the slots of the blocks
//     list[off[e] .. off[e+1]) (B slots each).
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"

namespace mx {

struct KMapGrouped {
  const int32_t* list;   // null: plain K range [0, K)
  int b0, blk;
  int64_t K;
  __device__ __forceinline__ void operator()(int s, int64_t& kc, int& kv) const {
    const int64_t q = int64_t(s) * kBK;
    if (list) {
      kc = int64_t(list[b0 + int(q / blk)]) * blk + q % blk;
      kv = kBK;
    } else {
      kc = q;
      const int64_t rem = K - q;
      kv = rem < kBK ? int(rem) : kBK;
    }
  }
};

template <int BM, int BN, int FA, int FB, bool SALIGN>
__global__ void __launch_bounds__(kThreads) gemm_store_kernel(GemmStoreArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * kBK];
  constexpr int FM = BM / 64, FN = BN / 64;
  const int per_group = p.tiles_m * p.tiles_n;
  const int tile = blockIdx.x;
  const int g = tile / per_group;
  const int t = tile - g * per_group;
  const int tm = t / p.tiles_n, tn = t - (t / p.tiles_n) * p.tiles_n;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  TileOperands<BM, BN, SALIGN> op;
#pragma unroll
  for (int q = 0; q < BM / 32; ++q) {
    const int64_t row = m0 + (threadIdx.x >> 3) + 32 * q;
    op.a.row[q] = row < p.M ? p.a_codes + row * p.lda : nullptr;
  }
#pragma unroll
  for (int q = 0; q < BN / 32; ++q) {
    const int64_t row = n0 + (threadIdx.x >> 3) + 32 * q;
    op.b.row[q] = row < p.N ? p.b_codes + row * p.ldb : nullptr;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = m0 + (wave >> 1) * (BM / 2) + i * 32 + (lane & 31);
    op.sa.row[i] = row < p.M ? p.a_scales + row * (p.lda / 32) : nullptr;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t row = n0 + (wave & 1) * (BN / 2) + j * 32 + (lane & 31);
    op.sb.row[j] = row < p.N ? p.b_scales + row * (p.ldb / 32) : nullptr;
  }
  KMapGrouped km{p.blk_list, 0, p.blk, p.K};
  int nstages;
  if (p.blk_list) {
    km.b0 = p.blk_off[g];
    nstages = int((int64_t(p.blk_off[g + 1] - km.b0) * p.blk) / kBK);
  } else {
    nstages = int((p.K + kBK - 1) / kBK);
  }
  v16f acc[FM][FN];
  mx_mainloop<BM, BN, FA, FB, SALIGN>(op, nstages, km, smem, acc);

  uint16_t* out = p.out + int64_t(g) * p.out_gstride;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + acc_col<BM, BN>(j);
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + acc_row<BM, BN>(i, q);
        if (row < p.M) out[row * p.ldo + col] = f32_to_bf16(acc[i][j][q]);
      }
    }
}

template <int BM, int BN, bool SALIGN>
static void launch_fmt(const GemmStoreArgs& p, int fa, int fb, unsigned blocks, hipStream_t st) {
  if (fa == 0 && fb == 0) gemm_store_kernel<BM, BN, 0, 0, SALIGN><<<blocks, kThreads, 0, st>>>(p);
  else if (fa == 0) gemm_store_kernel<BM, BN, 0, 1, SALIGN><<<blocks, kThreads, 0, st>>>(p);
  else if (fb == 0) gemm_store_kernel<BM, BN, 1, 0, SALIGN><<<blocks, kThreads, 0, st>>>(p);
  else gemm_store_kernel<BM, BN, 1, 1, SALIGN><<<blocks, kThreads, 0, st>>>(p);
}

hipError_t launch_gemm_store(GemmStoreArgs p, int groups, int fa, int fb, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0 || groups <= 0) return hipSuccess;
  // Larger tiles once there are enough of them to fill the chip (256 CUs).
  const bool big = (p.M >= 256 && p.N >= 256 &&
                    ((p.M + 255) / 256) * ((p.N + 255) / 256) * int64_t(groups) >= 224);
  const int BM = big ? 256 : 128, BN = big ? 256 : 128;
  p.tiles_m = int((p.M + BM - 1) / BM);
  p.tiles_n = int((p.N + BN - 1) / BN);
  const unsigned blocks = unsigned(int64_t(p.tiles_m) * p.tiles_n * groups);
  const bool salign = (p.lda % kBK == 0) && (p.ldb % kBK == 0);
  if (big) {
    if (salign) launch_fmt<256, 256, true>(p, fa, fb, blocks, st);
    else launch_fmt<256, 256, false>(p, fa, fb, blocks, st);
  } else {
    if (salign) launch_fmt<128, 128, true>(p, fa, fb, blocks, st);
    else launch_fmt<128, 128, false>(p, fa, fb, blocks, st);
  }
  return hipGetLastError();
}

}  // namespace mx
