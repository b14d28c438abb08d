// moe_aux.hip -- the HBM-bound kernels around the MoE GEMMs (gfx950):
// routing blocks, per-slot routing info, per-expert block lists, the
// token-axis quantised SwiGLU intermediate, the bias reductions and the
// finalisation of the fp32 accumulators into bf16 gradients.
//
// Routing blocks: P1 ("Blockwise MM Backward MXFP8 Kernel API Reference")
// parameters token_position_to_id [N*B] and block_to_expert [N].
// Bias reductions: P3 (sonic-moe functional/backward.py) db2_and_ds_kernel
// (db2 = sum of a*dY over an expert's slots; the <dY, b2> term of d(a)) and
// db1_kernel (db1 = sum of the gate/up gradients).
#include <mutex>

#include "kernels.hpp"
#include "moe_tiles.hpp"
#include "mx_device.hpp"
#include "swiglu.hpp"

namespace mx {

// ---------------------------------------------------------------------------
// small fills (plain kernels, so they are safe inside captured graphs)
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void fill_u16_kernel(uint16_t* p, int64_t n, uint16_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u16(void* p, int64_t n, uint16_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  fill_u16_kernel<<<unsigned(want < 8192 ? want : 8192), 256, 0, st>>>(static_cast<uint16_t*>(p), n, v);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  fill_u32_kernel<<<unsigned(want < 8192 ? want : 8192), 256, 0, st>>>(static_cast<uint32_t*>(p), n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// moe_build_blocks: the tokens are cut into C chunks of CH tokens (CH a
// multiple of 256, C at most route_max_chunks(E)).  The count kernel writes
// cnt[e * C + c], the tokens of chunk c routed to expert e; one workgroup turns
// the totals into each expert's first slot first[e] (its first block times B)
// and the block -> expert map; the place kernel then puts chunk c's tokens of
// expert e, ascending, from first[e] + (e's tokens in chunks before c) on.
// (One workgroup per expert scanning all tokens took 80 us of the large
// workload's step.)  A token is routed to e when any of its K ids is e;
// negative ids (dropped selections) and ids >= E match nothing.
//
// Chunks: one per 256 tokens up to kRouteChunkCap, with E * C at most
// kRouteCells (the workspace: counts plus first slots, 2 * kRouteCells words
// at most): more chunks, more workgroups in the count and place kernels.
constexpr int64_t kRouteChunkCap = 256;
constexpr int64_t kRouteCells = 4096 * 32;
static int64_t route_max_chunks(int64_t E) {
  const int64_t c = kRouteCells / E;
  return c < 1 ? 1 : (c > kRouteChunkCap ? kRouteChunkCap : c);
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* lds /*[4]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < 4; ++w) {
    const int s = lds[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// token t of a chunk routed to expert e?
__device__ __forceinline__ int routed_to(const int32_t* __restrict__ topk, int64_t t, int K, int e) {
  int hit = 0;
  for (int k = 0; k < K; ++k) hit |= topk[t * K + k] == e;
  return hit;
}

__global__ void __launch_bounds__(256) route_count_kernel(const int32_t* __restrict__ topk, int64_t T, int K,
                                                          int64_t CH, int C, int32_t* __restrict__ cnt) {
  __shared__ int red[4];
  const int e = blockIdx.x, c = blockIdx.y;
  const int64_t t0 = int64_t(c) * CH, t1 = t0 + CH < T ? t0 + CH : T;
  int n = 0;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) n += routed_to(topk, t, K, e);
  int tot;
  block_exclusive_scan(n, red, &tot);
  if (threadIdx.x == 0) cnt[e * C + c] = tot;
}

// One workgroup: expert e's blocks start after ceil(n_q / B) blocks of every
// q < e, n_q the total over the chunks; first[e] = that block times B; b2e of
// the used blocks.
__global__ void __launch_bounds__(256) route_offsets_kernel(const int32_t* __restrict__ cnt, int E, int C, int B,
                                                            int32_t* __restrict__ first, int32_t* __restrict__ b2e) {
  __shared__ int red[4];
  int blk = 0;   // first block of the current expert chunk
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + threadIdx.x;
    int n = 0;
    if (e < E) {
#pragma unroll 8
      for (int c = 0; c < C; ++c) n += cnt[e * C + c];
    }
    const int nb = (n + B - 1) / B;
    int tot;
    const int f = blk + block_exclusive_scan(nb, red, &tot);
    if (e < E) {
      first[e] = f * B;
      for (int q = 0; q < nb; ++q) b2e[f + q] = e;
    }
    blk += tot;
  }
}

__global__ void __launch_bounds__(256) route_place_kernel(const int32_t* __restrict__ topk, int64_t T, int K,
                                                          int64_t CH, int C, const int32_t* __restrict__ cnt,
                                                          const int32_t* __restrict__ first,
                                                          int32_t* __restrict__ tpid) {
  __shared__ int red[4];
  const int e = blockIdx.x, c = blockIdx.y;
  const int64_t t0 = int64_t(c) * CH, t1 = t0 + CH < T ? t0 + CH : T;
  int before;   // e's tokens in the chunks before c, summed over the workgroup
  {
    int n = 0;
    for (int q = threadIdx.x; q < c; q += 256) n += cnt[e * C + q];
    block_exclusive_scan(n, red, &before);
  }
  int64_t base = first[e] + before;
  for (int64_t tb = t0; tb < t1; tb += 256) {
    const int64_t t = tb + threadIdx.x;
    const int hit = t < t1 ? routed_to(topk, t, K, e) : 0;
    int tot;
    const int pos = block_exclusive_scan(hit, red, &tot);
    if (hit) tpid[base + pos] = int32_t(t);
    base += tot;
  }
}

// With E <= kRouteLdsExperts, one workgroup per chunk handles every expert:
// it counts with an LDS histogram, then places its tokens 256 at a time, each
// token finding its rank among the round's tokens of the same expert from a
// per-expert bitmap of the round in LDS (tokens ascending, as above).  Every
// chunk's ids are then read once per kernel instead of once per expert.
constexpr int kRouteLdsExperts = 1024;

// the token's expert at selection k, or -1: out of range, dropped, or a
// repeat of an earlier selection of the same token (counted once, as above)
__device__ __forceinline__ int route_sel(const int32_t* __restrict__ ids, int K, int k, int E) {
  const int e = ids[k];
  if (e < 0 || e >= E) return -1;
  for (int j = 0; j < k; ++j)
    if (ids[j] == e) return -1;
  return e;
}

// The same for a token whose K <= kRouteRegK ids sit in registers.
constexpr int kRouteRegK = 16;
__device__ __forceinline__ int route_sel_reg(const int (&ids)[kRouteRegK], int k, int E) {
  const int e = ids[k];
  if (e < 0 || e >= E) return -1;
  for (int j = 0; j < k; ++j)
    if (ids[j] == e) return -1;
  return e;
}

__global__ void __launch_bounds__(256) route_count_lds_kernel(const int32_t* __restrict__ topk, int64_t T, int K,
                                                              int64_t CH, int C, int E, int32_t* __restrict__ cnt) {
  __shared__ int hist[kRouteLdsExperts];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t t0 = int64_t(c) * CH, t1 = t0 + CH < T ? t0 + CH : T;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) {
    if (K <= kRouteRegK) {
      int ids[kRouteRegK];
      for (int k = 0; k < K; ++k) ids[k] = topk[t * K + k];
      for (int k = 0; k < K; ++k) {
        const int e = route_sel_reg(ids, k, E);
        if (e >= 0) atomicAdd(&hist[e], 1);
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const int e = route_sel(topk + t * K, K, k, E);
        if (e >= 0) atomicAdd(&hist[e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) cnt[e * C + c] = hist[e];
}

__global__ void __launch_bounds__(256) route_place_lds_kernel(const int32_t* __restrict__ topk, int64_t T, int K,
                                                              int64_t CH, int C, int E,
                                                              const int32_t* __restrict__ cnt,
                                                              const int32_t* __restrict__ first,
                                                              int32_t* __restrict__ tpid) {
  __shared__ uint32_t bits[kRouteLdsExperts][8];   // [expert][round token / 32]
  __shared__ int run[kRouteLdsExperts];            // next slot of (expert, this chunk)
  const int c = blockIdx.x, tid = threadIdx.x;
  // first slots: first[e] plus the counts of the chunks before c.  With E <
  // 256, tpe = 256 / E (a power of two) consecutive lanes share an expert,
  // each summing every tpe-th of those counts, then adding up across the lanes.
  {
    int tpe = 1;
    while (tpe * 2 * E <= 256 && tpe < 64) tpe *= 2;
    for (int e0 = 0; e0 < E; e0 += 256 / tpe) {
      const int e = e0 + tid / tpe, j = tid % tpe;
      int n = 0;
      if (e < E) {
#pragma unroll 8
        for (int q = j; q < c; q += tpe) n += cnt[e * C + q];
      }
      for (int o = 1; o < tpe; o <<= 1) n += __shfl_xor(n, o, 64);
      if (e < E && j == 0) run[e] = first[e] + n;
    }
  }
  __syncthreads();
  const int64_t t0 = int64_t(c) * CH, t1 = t0 + CH < T ? t0 + CH : T;
  for (int64_t tb = t0; tb < t1; tb += 256) {
    for (int i = tid; i < E * 8; i += 256) bits[i >> 3][i & 7] = 0u;
    __syncthreads();
    const int64_t t = tb + tid;
    const bool live = t < t1;
    const bool reg = K <= kRouteRegK;
    int ids[kRouteRegK];
    if (live && reg)
      for (int k = 0; k < K; ++k) ids[k] = topk[t * K + k];
    if (live)
      for (int k = 0; k < K; ++k) {
        const int e = reg ? route_sel_reg(ids, k, E) : route_sel(topk + t * K, K, k, E);
        if (e >= 0) atomicOr(&bits[e][tid >> 5], 1u << (tid & 31));
      }
    __syncthreads();
    if (live)
      for (int k = 0; k < K; ++k) {
        const int e = reg ? route_sel_reg(ids, k, E) : route_sel(topk + t * K, K, k, E);
        if (e >= 0) {
          int rank = __popc(bits[e][tid >> 5] & ((1u << (tid & 31)) - 1u));
          for (int w = 0; w < (tid >> 5); ++w) rank += __popc(bits[e][w]);
          tpid[run[e] + rank] = int32_t(t);
        }
      }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      int n = 0;
      for (int w = 0; w < 8; ++w) n += __popc(bits[e][w]);
      run[e] += n;
    }
    __syncthreads();
  }
}

int64_t build_blocks_workspace_bytes(int64_t E) { return E > 0 ? 2 * E * route_max_chunks(E) * 4 : 0; }

// The allocation-free variant's scratch: the counts and first slots per
// (expert, token chunk) for up to kNoAllocMaxExperts experts, 1 MiB per GPU,
// held from the library's load until the process ends.  Every word the three
// routing kernels read is written by an earlier one in the same call, so the
// array needs no clearing; calls that overlap on one GPU share it and race.
constexpr int64_t kNoAllocMaxExperts = 4096;
static __device__ __align__(256) int32_t scratch[2 * kRouteCells];
static_assert(sizeof(scratch) == (1 << 20), "scratch size");
static_assert(kNoAllocMaxExperts * 32 == kRouteCells, "the workspace of up to kNoAllocMaxExperts experts fits");

int64_t build_blocks_noalloc_max_experts() { return kNoAllocMaxExperts; }

// Device address of `scratch` on `device`, looked up once per device with that
// device current (each GPU holds its own copy at its own address) and kept.
// Host code never passes the array's name to a kernel: in host code it is a
// host-side stand-in, not a device address.
hipError_t build_blocks_scratch(int device, int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* ptrs[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[device] = static_cast<int32_t*>(p);
  }
  *out = ptrs[device];
  return hipSuccess;
}

hipError_t launch_build_blocks(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B, int64_t N,
                               int32_t* tpid, int32_t* b2e, int32_t* ws, hipStream_t st) {
  hipError_t err;
  if ((err = launch_fill_u32(tpid, N * B, 0xffffffffu, st)) != hipSuccess) return err;
  if ((err = launch_fill_u32(b2e, N, uint32_t(E - 1), st)) != hipSuccess) return err;
  if (T <= 0) return hipSuccess;
  // chunks of a multiple of 256 tokens, at most route_max_chunks(E) of them
  const int64_t cmax = route_max_chunks(E);
  const int64_t per = (T + cmax - 1) / cmax;
  const int64_t CH = (per + 255) / 256 * 256;
  const int C = int((T + CH - 1) / CH);
  int32_t* cnt = ws;               // [E][C]
  int32_t* first = ws + E * C;     // [E]; E * C + E <= 2 * E * cmax
  if (E <= kRouteLdsExperts) {
    route_count_lds_kernel<<<unsigned(C), 256, 0, st>>>(topk, T, int(K), CH, C, int(E), cnt);
    route_offsets_kernel<<<1, 256, 0, st>>>(cnt, int(E), C, int(B), first, b2e);
    route_place_lds_kernel<<<unsigned(C), 256, 0, st>>>(topk, T, int(K), CH, C, int(E), cnt, first, tpid);
    return hipGetLastError();
  }
  route_count_kernel<<<dim3(unsigned(E), unsigned(C)), 256, 0, st>>>(topk, T, int(K), CH, C, cnt);
  route_offsets_kernel<<<1, 256, 0, st>>>(cnt, int(E), C, int(B), first, b2e);
  route_place_kernel<<<dim3(unsigned(E), unsigned(C)), 256, 0, st>>>(topk, T, int(K), CH, C, cnt, first, tpid);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-slot routing info: token (-1 for padding or an invalid block expert) and
// affinity (0 for padding), and the inverse map slot_of[t*E + e] = the slot
// of pair (t, e) (a pair occupies at most one slot; -1 where none, filled
// beforehand).  Outside [0,T) is padding, and with a device count of valid
// tokens (P1's num_valid_tokens: the real tokens are the leading rows, a count
// above T means T) so is every token at or past it.
__global__ void slot_info_kernel(const int32_t* __restrict__ tpid, const int32_t* __restrict__ b2e,
                                 const float* __restrict__ aff, int64_t T, int64_t E, int64_t B, int64_t P,
                                 const int32_t* __restrict__ nvalid, int32_t* __restrict__ slot_tok,
                                 float* __restrict__ slot_aff, int32_t* __restrict__ slot_of) {
  const int64_t n = nvalid ? int64_t(*nvalid) : T;
  const int64_t Tv = n < 0 ? 0 : (n < T ? n : T);
  for (int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; s < P; s += int64_t(gridDim.x) * blockDim.x) {
    const int64_t e = b2e[s / B];
    const int64_t t = tpid[s];
    const bool ok = t >= 0 && t < Tv && e >= 0 && e < E;
    slot_tok[s] = ok ? int32_t(t) : -1;
    slot_aff[s] = ok ? aff[t * E + e] : 0.f;
    if (ok) slot_of[t * E + e] = int32_t(s);
  }
}

// A block's extent: one past its last routed slot (0: no routed slot, the block
// takes no part in the GEMMs).  Slots at or past the extent are padding, so
// the GEMMs skip tiles that start there.
__global__ void __launch_bounds__(256) block_flag_kernel(const int32_t* __restrict__ slot_tok, int64_t B,
                                                         int32_t* __restrict__ flag) {
  __shared__ int red[4];
  int ext = 0;
  for (int64_t p = threadIdx.x; p < B; p += 256)
    if (slot_tok[int64_t(blockIdx.x) * B + p] >= 0) ext = int(p) + 1;   // p ascends per thread
  for (int o = 32; o > 0; o >>= 1) ext = max(ext, __shfl_xor(ext, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ext;
  __syncthreads();
  if (threadIdx.x == 0) flag[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Per-expert lists of occupied blocks in ascending order: counts (one
// workgroup per expert, coalesced scans of the blocks), offsets (one
// workgroup), then each expert's list in block order (one workgroup each).
__global__ void __launch_bounds__(256) expert_count_kernel(const int32_t* __restrict__ b2e,
                                                           const int32_t* __restrict__ flag, int N,
                                                           int32_t* __restrict__ cnt) {
  __shared__ int red[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int b = threadIdx.x; b < N; b += 256) c += (b2e[b] == e) & (flag[b] != 0);
  int tot;
  block_exclusive_scan(c, red, &tot);
  if (threadIdx.x == 0) cnt[e] = tot;
}

__global__ void __launch_bounds__(256) expert_offsets_kernel(const int32_t* __restrict__ cnt, int E,
                                                             int32_t* __restrict__ off) {
  __shared__ int red[4];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + threadIdx.x;
    int tot;
    const int pos = block_exclusive_scan(e < E ? cnt[e] : 0, red, &tot) + carry;
    if (e < E) off[e] = pos;
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[E] = carry;
}

__global__ void __launch_bounds__(256) expert_list_kernel(const int32_t* __restrict__ b2e,
                                                          const int32_t* __restrict__ flag, int N,
                                                          const int32_t* __restrict__ off, int32_t* __restrict__ list) {
  __shared__ int red[4];
  const int e = blockIdx.x;
  int w = off[e];
  for (int b0 = 0; b0 < N; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int hit = b < N && b2e[b] == e && flag[b] != 0;
    int tot;
    const int pos = block_exclusive_scan(hit, red, &tot);
    if (hit) list[w + pos] = b;
    w += tot;
  }
}

// Tile ranges of a slot-blocked GEMM (see moe_tiles.hpp): start[b] = sum over
// blocks before b of ceil(extent / W) * other; start[N] = the total.  Then the
// tile -> block map start[N + 1 + t] = b for every tile t of block b, so a
// GEMM workgroup finds its block with one load instead of a binary search
// (a dozen dependent loads before its first DMA).  One workgroup.
__global__ void __launch_bounds__(256) tile_ranges_kernel(const int32_t* __restrict__ ext, int N, int W, int other,
                                                          int32_t* __restrict__ start, TailCut* __restrict__ cut,
                                                          int conc, int npairs, int rr, int cmax) {
  // With rr, the blocks whose slot tiles are all live (cmax tiles) come first,
  // in block order, and the partly filled ones after them: every round of
  // tiles then covers whole blocks of one expert (moe_tiles.hpp).
  __shared__ int red[4];
  __shared__ int carry_full, carry_part;
  if (threadIdx.x == 0) carry_full = carry_part = 0;
  __syncthreads();
  for (int b0 = 0; b0 < N; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int c = b < N ? (ext[b] + W - 1) / W * other : 0;
    const bool full = rr && c == cmax;
    int tot_full = 0, tot_part;
    const int pos_full = rr ? block_exclusive_scan(full ? c : 0, red, &tot_full) + carry_full : 0;   // rr: uniform
    const int pos_part = block_exclusive_scan(full ? 0 : c, red, &tot_part) + carry_part;
    if (b < N) start[b] = full ? pos_full : pos_part;   // partly filled blocks: relative for now
    __syncthreads();
    if (threadIdx.x == 0) {
      carry_full += tot_full;
      carry_part += tot_part;
    }
    __syncthreads();
  }
  const int total = carry_full + carry_part;
  // partly filled blocks after the full ones
  for (int b = threadIdx.x; b < N; b += 256) {
    const int c = (ext[b] + W - 1) / W * other;
    if (!(rr && c == cmax)) start[b] += carry_full;
  }
  if (threadIdx.x == 0) {
    start[N] = total;
    if (cut) {   // the tail cut of each XCD
      int base = 0;
      for (int x = 0; x < 8; ++x) {
        TailCut tc = tail_cut_one(total, x, rr, conc, npairs);
        tc.base = base;
        base += tc.tail * (tc.S - 1);
        cut[x] = tc;
      }
    }
  }
  __syncthreads();   // the starts written above are visible to the whole workgroup
  int32_t* map = start + N + 1;
  for (int b = threadIdx.x; b < N; b += 256) {
    const int t0 = start[b], c = (ext[b] + W - 1) / W * other;
    for (int t = t0; t < t0 + c; ++t) map[t] = b;
  }
}

hipError_t launch_tile_ranges(const int32_t* ext, int64_t N, int W, int other, int32_t* start, hipStream_t st,
                              TailCut* cut, int conc, int npairs, int rr, int blk) {
  const int cmax = (blk + W - 1) / W * other;   // tiles of a block whose slot tiles are all live
  tile_ranges_kernel<<<1, 256, 0, st>>>(ext, int(N), W, other, start, cut, conc, npairs, rr, cmax);
  return hipGetLastError();
}

hipError_t launch_slot_setup(const int32_t* tpid, const int32_t* b2e, const float* aff, int64_t T, int64_t E,
                             int64_t N, int64_t B, const int32_t* nvalid, int32_t* slot_tok, float* slot_aff,
                             int32_t* slot_of, int32_t* flag, int32_t* off, int32_t* list, hipStream_t st) {
  const int64_t P = N * B;
  const int64_t want = (P + 255) / 256;
  hipError_t err = launch_fill_u32(reinterpret_cast<uint32_t*>(slot_of), T * E, 0xffffffffu, st);
  if (err != hipSuccess) return err;
  slot_info_kernel<<<unsigned(want < 4096 ? want : 4096), 256, 0, st>>>(tpid, b2e, aff, T, E, B, P, nvalid,
                                                                           slot_tok, slot_aff, slot_of);
  block_flag_kernel<<<unsigned(N), 256, 0, st>>>(slot_tok, B, flag);
  // the counts go to off[1..E] and become offsets in place: in each 256-expert
  // chunk every count is read before the scan's barrier and every offset
  // written after it, and a chunk writes only indices the later chunks do not read
  expert_count_kernel<<<unsigned(E), 256, 0, st>>>(b2e, flag, int(N), off + 1);
  expert_offsets_kernel<<<1, 256, 0, st>>>(off + 1, int(E), off);
  expert_list_kernel<<<unsigned(E), 256, 0, st>>>(b2e, flag, int(N), off, list);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias terms (has_bias): per slot <dY_t, b2[e]> stored in daff_slot (one wave
// per slot), and db2[e][h] += sum over a block's slots of a * dY[t][h].
// H % 32 == 0 and dY / b2 rows 16-byte aligned: 8 values per lane and load.
__global__ void __launch_bounds__(256) bias_dot_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ b2,
                                                       const int32_t* __restrict__ slot_tok,
                                                       const int32_t* __restrict__ b2e, int64_t H, int64_t B,
                                                       int64_t P, float* __restrict__ daff_slot) {
  const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= P) return;
  const int64_t t = slot_tok[s];
  if (t < 0) return;
  const int64_t e = b2e[s / B];
  const uint4* yr = reinterpret_cast<const uint4*>(dy + t * H);
  const uint4* br = reinterpret_cast<const uint4*>(b2 + e * H);
  float acc = 0.f;
  for (int64_t c = lane; c < H / 8; c += 64) {
    const uint4 y = yr[c], w = br[c];
    const uint32_t ya[4] = {y.x, y.y, y.z, y.w}, wa[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += lo_bf16(ya[k]) * lo_bf16(wa[k]) + hi_bf16(ya[k]) * hi_bf16(wa[k]);
  }
  acc = wave_sum_xor(acc, 64);
  if (lane == 0) daff_slot[s] = acc;   // the slot's <dY, b2> term
}

// db2 of one block: thread = two adjacent columns h (4-byte loads), eight
// independent chains over the block's slots keep eight loads in flight; one
// atomic per (block, column).
__global__ void __launch_bounds__(256) db2_kernel(const uint16_t* __restrict__ dy, const int32_t* __restrict__ slot_tok,
                                                  const float* __restrict__ slot_aff, const int32_t* __restrict__ b2e,
                                                  const int32_t* __restrict__ flag, int64_t H, int64_t B,
                                                  float* __restrict__ db2_acc) {
  const int64_t b = blockIdx.y;
  const int64_t h = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 2;
  if (!flag[b] || h >= H) return;
  const int64_t e = b2e[b];
  float lo[8] = {}, hi[8] = {};
  for (int64_t p = 0; p < B; p += 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t t = slot_tok[b * B + p + k];
      if (t >= 0) {
        const float a = slot_aff[b * B + p + k];
        const uint32_t y = *reinterpret_cast<const uint32_t*>(dy + t * H + h);
        lo[k] += a * lo_bf16(y);
        hi[k] += a * hi_bf16(y);
      }
    }
  }
  atomicAdd(db2_acc + e * H + h, ((lo[0] + lo[1]) + (lo[2] + lo[3])) + ((lo[4] + lo[5]) + (lo[6] + lo[7])));
  atomicAdd(db2_acc + e * H + h + 1, ((hi[0] + hi[1]) + (hi[2] + hi[3])) + ((hi[4] + hi[5]) + (hi[6] + hi[7])));
}

hipError_t launch_bias(const uint16_t* dy, const uint16_t* b2, const int32_t* slot_tok, const float* slot_aff,
                       const int32_t* b2e, const int32_t* flag, int64_t H, int64_t B, int64_t N, float* daff_slot,
                       float* db2_acc, hipStream_t st) {
  const int64_t P = N * B;
  bias_dot_kernel<<<unsigned((P + 3) / 4), 256, 0, st>>>(dy, b2, slot_tok, b2e, H, B, P, daff_slot);
  db2_kernel<<<dim3(unsigned((H + 511) / 512), unsigned(N)), 256, 0, st>>>(dy, slot_tok, slot_aff, b2e, flag, H, B,
                                                                          db2_acc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Finalisation: fp32 accumulators -> bf16 outputs; d(a) scattered to t*E+e.
// With ACC the output's old bf16 value is added before the one rounding.
template <bool ACC>
__global__ void f32_to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n / 4; i += int64_t(gridDim.x) * blockDim.x) {
    float4 v = reinterpret_cast<const float4*>(src)[i];
    if (ACC) {
      const uint2 o = reinterpret_cast<const uint2*>(dst)[i];
      v.x += bf16_to_f32(uint16_t(o.x)); v.y += bf16_to_f32(uint16_t(o.x >> 16));
      v.z += bf16_to_f32(uint16_t(o.y)); v.w += bf16_to_f32(uint16_t(o.y >> 16));
    }
    const uint32_t lo = uint32_t(f32_to_bf16(v.x)) | (uint32_t(f32_to_bf16(v.y)) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16(v.z)) | (uint32_t(f32_to_bf16(v.w)) << 16);
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(lo, hi);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = (n & ~int64_t(3)) + threadIdx.x;
    dst[i] = f32_to_bf16(src[i] + (ACC ? bf16_to_f32(dst[i]) : 0.f));
  }
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t st, bool accumulate) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n / 4 + 255) / 256 + 1;
  const unsigned grid = unsigned(want < 16384 ? want : 16384);
  if (accumulate) f32_to_bf16_kernel<true><<<grid, 256, 0, st>>>(src, dst, n);
  else f32_to_bf16_kernel<false><<<grid, 256, 0, st>>>(src, dst, n);
  return hipGetLastError();
}

// dX[t] = sum over t's routed slots, in expert order, of the slot's Phase-3 row
// (fp32), rounded to bf16; a token without slots gets zeros.  One workgroup
// per token; H % 32 == 0.  The token's slots are compacted into LDS 256
// experts at a time (a block scan keeps expert order), then each thread sums
// up to four 4-column groups over them.  The rows are read and dX is stored
// with the nontemporal hint (the rows are read once, dX is the final output):
// 7-10% faster for each.
template <bool ACC>
__global__ void __launch_bounds__(256) dx_reduce_kernel(const float* __restrict__ dx_slot,
                                                        const int32_t* __restrict__ slot_of, int64_t E, int64_t H,
                                                        uint16_t* __restrict__ dx) {
  __shared__ int red[4];
  __shared__ int32_t list[256];
  const int64_t t = blockIdx.x;
  const int32_t* so = slot_of + t * E;
  const int64_t C = H / 4;   // 4-column groups
  for (int64_t c0 = 0; c0 < C; c0 += 4 * 256) {
    float4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t e0 = 0; e0 < E; e0 += 256) {
      const int64_t e = e0 + threadIdx.x;
      const int32_t s = e < E ? so[e] : -1;
      int n;
      const int pos = block_exclusive_scan(s >= 0 ? 1 : 0, red, &n);
      if (s >= 0) list[pos] = s;
      __syncthreads();
      for (int k = 0; k < n; ++k) {
        const float4* row = reinterpret_cast<const float4*>(dx_slot + int64_t(list[k]) * H);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t c = c0 + threadIdx.x + 256 * j;
          if (c < C) {
            const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + c));
            const float4 v = make_float4(x[0], x[1], x[2], x[3]);
            acc[j].x += v.x; acc[j].y += v.y; acc[j].z += v.z; acc[j].w += v.w;
          }
        }
      }
      __syncthreads();   // the list is rewritten by the next chunk
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = c0 + threadIdx.x + 256 * j;
      if (c < C) {
        uint2* dst = reinterpret_cast<uint2*>(dx + t * H) + c;
        if (ACC) {   // the old value joins after the slot sum, before the one rounding
          const uint2 o = *dst;
          acc[j].x += bf16_to_f32(uint16_t(o.x)); acc[j].y += bf16_to_f32(uint16_t(o.x >> 16));
          acc[j].z += bf16_to_f32(uint16_t(o.y)); acc[j].w += bf16_to_f32(uint16_t(o.y >> 16));
        }
        store_nt(dst, make_uint2(bf16x2_pack(acc[j].x, acc[j].y), bf16x2_pack(acc[j].z, acc[j].w)));
      }
    }
  }
}

hipError_t launch_dx_reduce(const float* dx_slot, const int32_t* slot_of, int64_t T, int64_t E, int64_t H,
                            uint16_t* dx, hipStream_t st, bool accumulate) {
  if (T <= 0) return hipSuccess;
  if (accumulate) dx_reduce_kernel<true><<<unsigned(T), 256, 0, st>>>(dx_slot, slot_of, E, H, dx);
  else dx_reduce_kernel<false><<<unsigned(T), 256, 0, st>>>(dx_slot, slot_of, E, H, dx);
  return hipGetLastError();
}

// d(a) of each routed slot: its bias term (0 without a bias) plus the
// epilogue's partials over the rows i, to bf16 at t*E+e.  A workgroup takes 64
// slots; wave w sums partials w, w+4, ... (coalesced over the slots), and the
// four sums are added in wave order, so the result does not vary run to run.
__global__ void __launch_bounds__(256) daff_scatter_kernel(const float* __restrict__ daff_slot,
                                                           const float* __restrict__ daff_part, int64_t nparts,
                                                           const int32_t* __restrict__ slot_tok,
                                                           const int32_t* __restrict__ b2e, int64_t E, int64_t B,
                                                           int64_t P, int accumulate,
                                                           uint16_t* __restrict__ daff) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t s = int64_t(blockIdx.x) * 64 + lane;
  float acc = 0.f;
  if (s < P) {
#pragma unroll 8
    for (int64_t g = w; g < nparts; g += 4) acc += daff_part[g * P + s];
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0 && s < P) {
    const int64_t t = slot_tok[s];
    if (t >= 0) {
      float d = daff_slot[s] + ((part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]));
      uint16_t* dst = daff + t * E + b2e[s / B];
      if (accumulate) d += bf16_to_f32(*dst);
      *dst = f32_to_bf16(d);
    }
  }
}

hipError_t launch_daff_scatter(const float* daff_slot, const float* daff_part, int64_t nparts,
                               const int32_t* slot_tok, const int32_t* b2e, int64_t T, int64_t E, int64_t B,
                               int64_t N, uint16_t* daff, hipStream_t st, bool accumulate) {
  if (!accumulate) {   // pairs without a slot are 0; accumulating, they keep their value
    hipError_t err = launch_fill_u16(daff, T * E, 0, st);
    if (err != hipSuccess) return err;
  }
  const int64_t P = N * B;
  daff_scatter_kernel<<<unsigned((P + 63) / 64), 256, 0, st>>>(daff_slot, daff_part, nparts, slot_tok, b2e, E, B, P,
                                                                accumulate ? 1 : 0, daff);
  return hipGetLastError();
}

}  // namespace mx
