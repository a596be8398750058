// Compact block prefix-LM mask on gfx950.
//
// Rule ("VLA 代码精读" §1.2 and §1.5; "π0.5 vs MM-DiT joint attention", cumsum rule and
// three-block permission table; "Pi0-FAST 模型架构" §2.3): key j is visible from
// query i iff cumsum(ar)[j] <= cumsum(ar)[i], both tokens are valid, and the
// (segment(i), segment(j)) pair is not forbidden.  Instead of an N x N mask the
// builder emits one packed word per token and one class per 16x32 tile.
#include "common.h"

#include <algorithm>

namespace {

constexpr int kScanThreads = 1024;

// Inclusive scan of one int per thread across the block (64-lane waves).
__device__ int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int nw = blockDim.x >> 6;
    int t = lane < nw ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int u = __shfl_up(t, off);
      if (lane >= off) t += u;
    }
    if (lane < nw) wave_tot[lane] = t;
  }
  __syncthreads();
  int base = wave > 0 ? wave_tot[wave - 1] : 0;
  __syncthreads();
  return v + base;
}

// One block per sample: block ids (inclusive cumsum of ar), positions
// (cumsum of valid minus one) and packed token words.
__global__ void __launch_bounds__(kScanThreads)
mask_scan_kernel(const uint8_t* __restrict__ input_mask, const uint8_t* __restrict__ ar,
                 const uint8_t* __restrict__ seg, int N, int32_t* __restrict__ bid,
                 int32_t* __restrict__ pos, uint32_t* __restrict__ tok) {
  __shared__ int tot_a[16];
  __shared__ int tot_v[16];
  const int b = blockIdx.x;
  const int chunk = (N + kScanThreads - 1) / kScanThreads;
  const int lo = min(N, (int)threadIdx.x * chunk);
  const int hi = min(N, lo + chunk);
  const uint8_t* valid = input_mask + (size_t)b * N;
  int sa = 0, sv = 0;
  for (int i = lo; i < hi; ++i) {
    sa += ar[i] != 0;
    sv += valid[i] != 0;
  }
  int inc_a = block_inclusive_scan(sa, tot_a);
  int inc_v = block_inclusive_scan(sv, tot_v);
  int ca = inc_a - sa;  // exclusive prefix before this chunk
  int cv = inc_v - sv;
  for (int i = lo; i < hi; ++i) {
    ca += ar[i] != 0;
    int vi = valid[i] != 0;
    cv += vi;
    uint32_t sg = seg ? (uint32_t)(seg[i] & 3u) : 0u;
    if (b == 0) bid[i] = ca;
    pos[(size_t)b * N + i] = cv - 1;
    tok[(size_t)b * N + i] = (uint32_t)vi | (sg << 1) | ((uint32_t)ca << 3);
  }
}

// One wave per (b, query tile, key tile): classify the tile.  Lane l takes key
// k0 + l % 32 against the query rows q0 + l / 32 + 2r; ballots count the visible
// and in-range pairs.  A key tile that runs past N is never FULL, so the
// attention kernels always mask its padding.
static_assert(PI_MASK_TILE_K == 32 && PI_MASK_TILE_Q % 2 == 0, "mask_tiles_kernel maps 32 keys x 2 rows per pass");

__global__ void __launch_bounds__(256)
mask_tiles_kernel(const uint32_t* __restrict__ tok, int B, int N, int n_qt, int n_kt, uint32_t forbid,
                  uint8_t* __restrict__ tiles) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)B * n_qt * n_kt;
  if (id >= total) return;
  const int kt = (int)(id % n_kt);
  const int qt = (int)((id / n_kt) % n_qt);
  const int b = (int)(id / ((int64_t)n_kt * n_qt));
  const uint32_t* t = tok + (size_t)b * N;
  const int q0 = qt * PI_MASK_TILE_Q, q1 = min(N, q0 + PI_MASK_TILE_Q);
  const int k0 = kt * PI_MASK_TILE_K, k1 = min(N, k0 + PI_MASK_TILE_K);
  const int j = k0 + (lane & 31);
  const uint32_t wk = j < k1 ? t[j] : 0u;
  int vis = 0, pairs = 0;
#pragma unroll
  for (int r = 0; r < PI_MASK_TILE_Q / 2; ++r) {
    const int i = q0 + (lane >> 5) + 2 * r;
    const bool in = i < q1 && j < k1;
    const uint32_t wq = i < q1 ? t[i] : 0u;
    vis += __popcll(__ballot(in && pair_visible(wq, wk, forbid)));
    pairs += __popcll(__ballot(in));
  }
  if (lane == 0) {
    uint8_t cls = PI_TILE_PARTIAL;
    if (vis == 0) cls = PI_TILE_EMPTY;
    else if (vis == pairs && (k1 - k0) == PI_MASK_TILE_K) cls = PI_TILE_FULL;
    tiles[id] = cls;
  }
}

__global__ void mask_dense_kernel(const uint32_t* __restrict__ tok, int N, uint32_t forbid,
                                  int64_t total, uint8_t* __restrict__ dense) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int j = (int)(id % N);
  const int i = (int)((id / N) % N);
  const int b = (int)(id / ((int64_t)N * N));
  const uint32_t* t = tok + (size_t)b * N;
  dense[id] = pair_visible(t[i], t[j], forbid) ? 1 : 0;
}

struct MaskLayout {
  size_t bid, pos, tok, tiles, total;
  int n_qt, n_kt;
};

MaskLayout mask_layout(int B, int N) {
  MaskLayout L;
  L.n_qt = (N + PI_MASK_TILE_Q - 1) / PI_MASK_TILE_Q;
  L.n_kt = (N + PI_MASK_TILE_K - 1) / PI_MASK_TILE_K;
  size_t off = 0;
  L.bid = off; off = pi::align_up(off + sizeof(int32_t) * (size_t)N, 256);
  L.pos = off; off = pi::align_up(off + sizeof(int32_t) * (size_t)B * N, 256);
  L.tok = off; off = pi::align_up(off + sizeof(uint32_t) * (size_t)B * N, 256);
  L.tiles = off; off = pi::align_up(off + (size_t)B * L.n_qt * L.n_kt, 256);
  L.total = off;
  return L;
}

}  // namespace

extern "C" size_t pi_mask_workspace_bytes(int B, int N) {
  if (B < 1 || N < 1 || B > 65535 || N > (1 << 20)) return 0;
  return mask_layout(B, N).total;
}

extern "C" pi_status pi_mask_build(const uint8_t* input_mask, const uint8_t* ar, const uint8_t* seg,
                                   uint32_t forbid_bits, int B, int N, void* workspace,
                                   size_t workspace_bytes, pi_mask* out, pi_stream stream) {
  PI_REQUIRE(out && input_mask && ar && workspace, PI_ERR_INVALID_ARG, "pi_mask_build: null pointer");
  PI_REQUIRE(B >= 1 && B <= 65535 && N >= 1 && N <= (1 << 20), PI_ERR_INVALID_ARG,
             "pi_mask_build: B=%d N=%d out of range", B, N);
  PI_REQUIRE(forbid_bits <= 0xFFFFu, PI_ERR_INVALID_ARG, "pi_mask_build: forbid_bits uses segments >= 4");
  MaskLayout L = mask_layout(B, N);
  PI_REQUIRE(workspace_bytes >= L.total, PI_ERR_WORKSPACE, "pi_mask_build: workspace %zu < %zu bytes",
             workspace_bytes, L.total);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_mask_build: workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  pi_mask m;
  m.B = B;
  m.N = N;
  m.n_qt = L.n_qt;
  m.n_kt = L.n_kt;
  m.forbid_bits = forbid_bits;
  m.bid = reinterpret_cast<int32_t*>(ws + L.bid);
  m.pos = reinterpret_cast<int32_t*>(ws + L.pos);
  m.tok = reinterpret_cast<uint32_t*>(ws + L.tok);
  m.tiles = reinterpret_cast<uint8_t*>(ws + L.tiles);
  hipStream_t s = static_cast<hipStream_t>(stream);
  mask_scan_kernel<<<B, kScanThreads, 0, s>>>(input_mask, ar, seg, N, m.bid, m.pos, m.tok);
  pi_status st = pi::check_launch("mask_scan_kernel");
  if (st != PI_OK) return st;
  int64_t ntiles = (int64_t)B * L.n_qt * L.n_kt;
  const int64_t blocks = (ntiles + 3) / 4;   // four waves of 64 per workgroup, one tile each
  PI_REQUIRE(blocks < (1ll << 31), PI_ERR_UNSUPPORTED, "pi_mask_build: too many tiles");
  mask_tiles_kernel<<<(unsigned)blocks, 256, 0, s>>>(m.tok, B, N, L.n_qt, L.n_kt, forbid_bits, m.tiles);
  st = pi::check_launch("mask_tiles_kernel");
  if (st != PI_OK) return st;
  *out = m;
  return PI_OK;
}

extern "C" pi_status pi_mask_materialize(const pi_mask* mask, uint8_t* dense, pi_stream stream) {
  PI_REQUIRE(mask && dense && mask->tok, PI_ERR_INVALID_ARG, "pi_mask_materialize: null pointer");
  PI_REQUIRE(mask->B >= 1 && mask->N >= 1 && mask->N <= (1 << 16), PI_ERR_INVALID_ARG,
             "pi_mask_materialize: B=%d N=%d out of range (N <= 65536)", mask->B, mask->N);
  int64_t total = (int64_t)mask->B * mask->N * mask->N;
  int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  PI_REQUIRE(blocks < (1ll << 31), PI_ERR_INVALID_ARG, "pi_mask_materialize: too large");
  mask_dense_kernel<<<(unsigned)blocks, threads, 0, static_cast<hipStream_t>(stream)>>>(
      mask->tok, mask->N, mask->forbid_bits, total, dense);
  return pi::check_launch("mask_dense_kernel");
}
