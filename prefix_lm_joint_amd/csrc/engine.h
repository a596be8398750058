// Pieces of the gfx950 attention engine shared by the forward and backward
// kernels: key tile size, the swizzled LDS tile and its direct-to-LDS buffer
// loads, the transposing LDS read and the XCD-aware workgroup placement.
#pragma once

#include "common.h"

namespace pi_engine {

constexpr int TK = 32;             // keys per tile
constexpr int kMaxTiles = 512;     // longest key sequence a workgroup walks: 16384 tokens

#define PI_LDS __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

extern "C" __device__ void pi_buffer_load_lds(i32x4 rsrc, PI_LDS uint32_t* lds, int size, int voffset, int soffset,
                                              int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer resource over [base, base + 2 GiB): any offset >= 0x7FFFFFFF reads as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base) {
  struct __attribute__((packed)) Res {
    const void* p;
    uint32_t range;
    uint32_t cfg;
  } r{base, 0x7FFFFFFFu, 0x00020000u};
  i32x4 v = __builtin_bit_cast(i32x4, r);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_readfirstlane(v[i]);
  return v;
}
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ PI_LDS uint32_t* lds_u32(const void* p) {
  return (PI_LDS uint32_t*)(const_cast<void*>(p));
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0 only).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read of 4 bf16 (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane i receives element i % 4 of the 4 elements addressed by lanes
// 4k + i/4, k = 0..3: lanes pointed at 4 rows x 16 columns of a row-major tile
// (lane j at row j/4, columns 4(j%4)..) hand lane i column i of those 4 rows.
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PI_LDS bf16x4*)(const_cast<__bf16*>(p)));
}

// ---------------------------------------------------------------------------
// Swizzled LDS tile.  A row holds D bf16 (CHR chunks of 16 bytes); logical chunk
// x of row r sits at physical chunk x ^ f(r).
//   K fragment read: 16 lanes read rows r0..r0+15 at one logical chunk.  d = 256:
//     f_K(r) = r & 15 spreads them over 16 distinct chunks (all 64 banks);
//     d = 64 (rows of 32 banks): f_K(r) = (r >> 1) & 7 does the same.
//   V transposing read: 16 lanes read 4 rows x 32 bytes (two chunks).
//     d = 256: f_V(r) = 2r & 31; d = 64: f_V(r) = r & 6; 32 lanes (8 rows) then
//     cover all 64 banks once.
// (The 32 x 32 x 16 engine's tiles, read both row-wise and transposed in the
// backward, use their own swizzle: attention32.hip.)
// ---------------------------------------------------------------------------
template <int D>
struct Tile {
  static constexpr int CHR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CHR;              // rows per 64-lane load instruction
  static constexpr int INSTS = TK / RPI;            // load instructions per tensor tile
  __device__ static __forceinline__ int fk(int r) { return D == 256 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int fv(int r) { return D == 256 ? ((2 * r) & 31) : (r & 6); }
};

template <int D>
struct Stage {
  alignas(16) __bf16 k[TK * D];
  alignas(16) __bf16 v[TK * D];
  alignas(16) uint32_t w[64];   // per-key mask words (lanes >= 32 land as zeros)
};

// This wave's share of the direct-to-LDS loads of one K/V tile: the per-lane
// byte offsets within a tile (row r of the tile at r * tsb, the row's swizzle
// folded in) are computed once; each tile then only moves the resource base.
// Per-lane offsets of the load wave's direct-to-LDS loads: instruction j of a
// tensor tile fetches rows j*RPI + lane/CHR, each lane one 16-byte chunk (its
// source chunk pre-swizzled so the LDS image comes out XOR-swizzled).
template <int D>
struct KvLanes {
  static constexpr int N = Tile<D>::INSTS;
  uint32_t k[N], v[N];
  int row[N];
};

// K with f_K, V with f_V.
template <int D>
__device__ __forceinline__ KvLanes<D> kv_lanes(int tsb) {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int p = lane % T::CHR;
  KvLanes<D> kl;
#pragma unroll
  for (int j = 0; j < KvLanes<D>::N; ++j) {
    const int r = j * T::RPI + lane / T::CHR;
    kl.row[j] = r;
    kl.k[j] = (uint32_t)r * (uint32_t)tsb + 16u * (uint32_t)(p ^ T::fk(r));
    kl.v[j] = (uint32_t)r * (uint32_t)tsb + 16u * (uint32_t)(p ^ T::fv(r));
  }
  return kl;
}

// All loads of the tile whose first key is key0 (k0, v0: key 0 of this sample
// and head; tsb bytes between consecutive keys), issued by the load wave.  Keys
// whose bit is clear in `keymask` (past the end, padding) are fetched from an
// out-of-range offset and land as zeros.
template <int D>
__device__ __forceinline__ void issue_kv(Stage<D>& st, const KvLanes<D>& kl, const __bf16* k0, const __bf16* v0,
                                         int key0, int tsb, uint32_t keymask) {
  using T = Tile<D>;
  const int64_t at = (int64_t)__builtin_amdgcn_readfirstlane(key0) * tsb;
  const bool full = __builtin_amdgcn_readfirstlane(keymask) == 0xFFFFFFFFu;
  const i32x4 rk = make_rsrc(reinterpret_cast<const char*>(k0) + at);
  const i32x4 rv = make_rsrc(reinterpret_cast<const char*>(v0) + at);
#pragma unroll
  for (int j = 0; j < KvLanes<D>::N; ++j) {
    uint32_t ok = kl.k[j], ov = kl.v[j];
    if (!full && !((keymask >> kl.row[j]) & 1u)) ok = ov = kOOB;
    pi_buffer_load_lds(rk, lds_u32(&st.k[j * T::RPI * D]), 16, (int)ok, 0, 0, 0);
    pi_buffer_load_lds(rv, lds_u32(&st.v[j * T::RPI * D]), 16, (int)ov, 0, 0, 0);
  }
}

// Workgroup placement.  Workgroups are dispatched round-robin over the 8 XCDs,
// each with its own L2.  With at least 8 groups, a group's workgroups (which read
// the same K/V) are kept on one XCD.  With fewer groups (one or a few samples,
// whose K/V are small) the workgroups simply go round-robin in group-major
// order, which spreads every group over all XCDs and keeps the XCDs balanced.
// Returns false for a workgroup with no work (the grid is rounded up).
struct Placement {
  int n_groups, n_sub;
  bool per_xcd;
};

__host__ __device__ inline Placement make_placement(int n_groups, int n_sub) {
  return Placement{n_groups, n_sub, n_groups >= 8};
}

__host__ inline int64_t placement_grid(const Placement& p) {
  return p.per_xcd ? (int64_t)((p.n_groups + 7) / 8 * 8) * p.n_sub : (int64_t)p.n_groups * p.n_sub;
}

__device__ __forceinline__ bool xcd_place(const Placement& p, int& group, int& sub) {
  const int id = blockIdx.x;
  if (!p.per_xcd) {
    group = id / p.n_sub;
    sub = id % p.n_sub;
    return group < p.n_groups;
  }
  const int xcd = id & 7;
  const int k = id >> 3;
  group = (k / p.n_sub) * 8 + xcd;
  sub = k % p.n_sub;
  return group < p.n_groups;
}

// bits[w] (w < n_words) = validity of tokens 32 w .. 32 w + 31 of one sample
// (bit j set: token 32 w + j < L and its word's valid bit is set); one ballot per
// 32 tokens, shared by the nwaves waves of the workgroup.  The token words of
// up to kBatch rounds are loaded before the first ballot needs one, so a whole
// row costs one memory latency, not one per round.
__device__ __forceinline__ void token_bitmap(const uint32_t* tk, int L, int n_words, int nwaves, uint32_t* bits) {
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int stride = nwaves * 64, end = n_words * TK;
  for (int base0 = wave * 64; base0 < end; base0 += kBatch * stride) {
    uint32_t w[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = base0 + u * stride + lane;
      w[u] = t < L ? tk[t] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int base = base0 + u * stride;
      if (base >= end) break;
      const unsigned long long bal = __ballot(w[u] & 1u);
      if (lane == 0) bits[base / TK] = (uint32_t)bal;
      if (lane == 32 && base / TK + 1 < n_words) bits[base / TK + 1] = (uint32_t)(bal >> 32);
    }
  }
}

// Setup of a query-major workgroup (all nwaves waves of it call this): kmask[kt]
// = validity bitmap of key tile kt of this sample (bit j: key 32 kt + j exists
// and is valid; one ballot per 32 keys), and, from wave 0, tlist[0 .. *tcount) =
// the key tiles holding a visible pair for query tokens [tok0, tok0 + ntok), each
// as tile | class << 16, the class merged over the 16-token query tiles those
// tokens span (kept where they agree, else PARTIAL).  trow: this sample's
// [n_qt, n_kt] tile classes.  Wave 0 loads the classes of the first two query
// tiles before the token words, so both arrive within one memory latency.  The
// caller synchronises before reading them.
__device__ __forceinline__ void query_block_tiles(const uint32_t* tk, int L, const uint8_t* trow, int n_qt, int n_kt,
                                                  int tok0, int ntok, int nwaves, uint32_t* kmask, uint32_t* tlist,
                                                  int* tcount) {
  constexpr int kC = kMaxTiles / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt_lo = tok0 / PI_MASK_TILE_Q;
  const int qt_hi = min(n_qt, (tok0 + ntok + PI_MASK_TILE_Q - 1) / PI_MASK_TILE_Q);
  int c0[kC], c1[kC];
  if (wave == 0) {
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int kt = u * 64 + lane;
      c0[u] = (kt < n_kt && qt_lo < qt_hi) ? trow[(size_t)qt_lo * n_kt + kt] : 0;
      c1[u] = (kt < n_kt && qt_lo + 1 < qt_hi) ? trow[(size_t)(qt_lo + 1) * n_kt + kt] : c0[u];
    }
  }
  token_bitmap(tk, L, n_kt, nwaves, kmask);
  if (wave != 0) return;
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kC; ++u) {
    if (u * 64 >= n_kt) break;
    const int kt = u * 64 + lane;
    int cls = 0;
    if (kt < n_kt) {
      cls = c0[u] == c1[u] ? c0[u] : PI_TILE_PARTIAL;
      for (int qt = qt_lo + 2; qt < qt_hi; ++qt) {   // a block spanning three or more query tiles
        const int cl = trow[(size_t)qt * n_kt + kt];
        cls = cls == cl ? cls : PI_TILE_PARTIAL;
      }
    }
    const unsigned long long bal = __ballot(cls > 0);
    if (cls > 0) tlist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (uint32_t)kt | ((uint32_t)cls << 16);
    cnt += __popcll(bal);
  }
  if (lane == 0) *tcount = cnt;
}

}  // namespace pi_engine
