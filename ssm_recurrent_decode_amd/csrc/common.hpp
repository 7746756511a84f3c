// Shared device/host helpers for the gfx950 decode kernels.
//
// Lane layout used by every state-streaming kernel ("tile layout")
// ------------------------------------------------------------------
// A per-head state is a d x n fp32 matrix stored row-major (n fastest).  It is cut
// into 16 x 16 tiles.  In a wave of 64 lanes, lane l owns row r = l & 15 of a row
// tile and the four consecutive columns 4*(l >> 4) .. +3 of every 16-column tile,
// loaded as one float4 per tile.  This is exactly the accumulator layout of
// v_mfma_f32_16x16x4_f32 when the MFMA computes the transposed tile (state columns
// on the M axis, state rows on the N axis), so a rank-c update S += V diag(w) K^T
// runs on the matrix cores straight from the registers the state was loaded into,
// and a row's dot product with a vector needs only a two-step reduction over the
// four lanes l, l^16, l^32, l^48 that share the row.
//
// Between HBM and that layout the state moves in the "line arrangement" (see
// load_state_lines below): every load or store instruction covers whole 128-byte
// lines, and it is non-temporal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssm_recurrent_decode.h"

namespace rssm {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v3u __attribute__((ext_vector_type(3)));

constexpr int kWave = 64;
constexpr int kBlock = 256;          // four waves per work-group
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxL = 32;            // ring capacity limit (entries fit one wave)
constexpr int kMaxT = 8;             // draft window limit
constexpr int kNumXcd = 8;           // MI355X: eight accelerator dies, one L2 each

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// softplus in fp32; above 20 the correction log1p(e^-x) is below fp32 resolution.
__device__ __forceinline__ float softplus_f32(float x) { return x > 20.f ? x : log1pf(expf(x)); }

// Work-groups are dispatched round-robin over the XCDs (block i -> XCD i % 8).
// Renumber so that each XCD receives chunks of kXcdChunk consecutive logical
// work-groups, the chunks dealt round-robin: neighbouring heads (a group's k/q and
// ring keys) meet in one L2, while all eight XCDs stream from the same region of
// the state at any time.  Measured against one contiguous eighth per XCD and
// against the plain dispatch order, interleaved launch by launch on the same
// buffers: chunks of 4 were fastest for the append (-6 %), GDN verify (-3.8 %)
// and standard step (-2.5 %); the Mamba-2 verify was 1 % faster still with the
// plain order.  Blocks past the largest multiple of 8 * kXcdChunk keep their id.
// The Mamba-2 append-decode takes chunks of 8 (two head blocks per XCD): -1.2 to
// -1.8 % per launch in two interleaved runs after the state moved as whole lines,
// fused front-end -0.5 %; chunks of 16: -0.3 %.  The verify kernels stay at 4
// (chunks of 8: Mamba-2 verify +0.5 %, GDN verify +1.7 %).
constexpr int kXcdChunk = 4;
constexpr int kXcdChunkAppend = 8;
template <int CH = kXcdChunk>
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int full = (nblocks / (kNumXcd * CH)) * (kNumXcd * CH);
  if (bid >= full) return bid;
  const int x = bid % kNumXcd, i = bid / kNumXcd;  // XCD, and dispatch order within it
  return ((i / CH) * kNumXcd + x) * CH + i % CH;
}

// Ring values (Mamba-2 v) and corrections (GDN u) of one slot are kept side by
// side for blocks of kXcdChunk consecutive heads: vu[rows][H / hb][L][hb][d],
// hb = ring_head_block(H).  The work-groups of a block run on one XCD at the
// same time (xcd_remap), so the entries one call caches for them form one
// contiguous span (4 x 128 bytes for d = 64 bf16) instead of lines 2 KB apart,
// and a head's c cached entries are read back at a stride of hb entries.
// Measured on the append-decode workload (B = 256, H = 32, d = 64, L = 16),
// interleaved against the per-head layout vu[rows][H][L][d] over whole ring
// cycles: -0.4 to -0.9 % per launch on three boxes (blocks of 8 and 16 heads
// the same, blocks of 2 no gain); the verify rows unchanged within 0.5 %.
__host__ __device__ constexpr int ring_head_block_log2(int H) { return H % 4 == 0 ? 2 : (H % 2 == 0 ? 1 : 0); }
static_assert(kXcdChunk == 4, "ring head blocks follow the XCD chunks");

// Element offset of slot `slot` of head h of pool row rb in the ring values or
// corrections (d elements per entry).
__device__ __forceinline__ size_t ring_entry(int rb, int h, int H, int L, int slot, int D) {
  const int sh = ring_head_block_log2(H);
  return ((((size_t)rb * (H >> sh) + (h >> sh)) * L + slot) << sh | (h & ((1 << sh) - 1))) * (size_t)D;
}

// Physical slot of logical ring entry j (0 <= j < L) when the oldest entry sits in
// slot head (0 <= head < L): head + j wraps at most once.
__device__ __forceinline__ int ring_slot(int head, int j, int L) {
  const int s = head + j;
  return s >= L ? s - L : s;
}

// ---- cross-lane steps in registers (DPP and the gfx950 lane swaps, no LDS)
// DPP controls of the gfx9 encoding.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;   // row_shr:n = 0x110 + n
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124;   // row_ror:n = 0x120 + n
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// src moved by the DPP pattern CTRL; lanes with no source, and lanes of rows not
// in ROW_MASK, get `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                    ROW_MASK, 0xF, false));
}

// Exclusive prefix product over the 64 lanes of a wave: returns
// prod_{l' < lane} x_{l'} and sets *all = prod over all lanes (every lane).
// Hillis-Steele steps inside each row of 16 lanes, then the row totals are
// carried across rows; products only, never a division, so an underflow to zero
// stays zero.  All lanes of the wave must be active.
__device__ __forceinline__ float prefix_product_excl(float x, float* all) {
  float v = x;
  v *= dpp_move<kDppRowShr1>(1.f, v);
  v *= dpp_move<kDppRowShr2>(1.f, v);
  v *= dpp_move<kDppRowShr4>(1.f, v);
  v *= dpp_move<kDppRowShr8>(1.f, v);
  v *= dpp_move<kDppRowBcast15, 0xA>(1.f, v);  // rows 1, 3 take lane 15 of rows 0, 2
  v *= dpp_move<kDppRowBcast31, 0xC>(1.f, v);  // rows 2, 3 take lane 31
  *all = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
  return dpp_move<kDppWaveShr1>(1.f, v);
}

// Sum over the four lanes that share a row in the tile layout (lanes l, l^16,
// l^32, l^48), every lane receiving the sum.
__device__ __forceinline__ float reduce_row4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(a[0]) + __int_as_float(a[1]);  // v_l + v_{l^16}
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(c[0]) + __int_as_float(c[1]);  // ... + the same from l^32
}

// Sum over the 16 lanes of a row, every lane of the row receiving the sum.
__device__ __forceinline__ float reduce_quarter(float v) {
  v += dpp_move<kDppRowRor8>(0.f, v);
  v += dpp_move<kDppRowRor4>(0.f, v);
  v += dpp_move<kDppQuadXor2>(0.f, v);
  v += dpp_move<kDppQuadXor1>(0.f, v);
  return v;
}

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void st_f4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ uint2 ld_u2(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint4 ld_u4(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// ---- a head's state between HBM and the tile layout
// In the tile layout one instruction moves 16 rows x 64 bytes, half of every
// 128-byte line it touches, and the other half comes with the next column tile.
// The state is therefore moved in the line arrangement instead: each pair of
// column tiles 2jj, 2jj + 1 (one 128-byte line per row) travels as two
// instructions, A with rows 0..7 of the row tile and B with rows 8..15, each
// covering its eight lines whole.  Lanes r < 8 carry the left halves (columns
// 32jj + 4cq ..) of row r in A and of row r + 8 in B; lanes r >= 8 the right
// halves (columns 32jj + 16 + 4cq ..) of row r - 8 in A and of row r in B.  One
// exchange between lanes r and r ^ 8 (settle_pair) turns a pair into the tile
// layout; the same exchange turns it back.  Loads and stores of the state are
// non-temporal: a launch touches each state byte once.  Measured interleaved on
// the same buffers, bit-identical results: append-decode -5.6 %, Mamba-2 verify
// (B = 512, T = 4) -10 %, GDN verify (B = 256, d = 128, T = 4) -16 %, fused
// front-end -4.7 % per launch against tile-layout transfers with plain loads and
// stores; non-temporal loads in the tile layout were 8 % slower, and the line
// arrangement with plain loads 1-4 % slower.
__device__ __forceinline__ float4 ld_f4_nt(const float* p) {
  const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_f4_nt(float* p, float4 v) {
  __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
}

// old with the lanes of the banks in BANKS (groups of four lanes of each row of
// 16: bank 0 = lanes 0..3, ...) replaced by src from the lane eight places away
// in the same row
template <int BANKS>
__device__ __forceinline__ float ror8_into(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kDppRowRor8, 0xF,
                                                    BANKS, false));
}

// A pair of column tiles between the line arrangement and the tile layout (the
// map is its own inverse): lanes r >= 8 take b of lane r - 8 into a, lanes r < 8
// take a of lane r + 8 into b.
__device__ __forceinline__ void settle_pair(float4& a, float4& b) {
  const float4 a0 = a, b0 = b;
  a = make_float4(ror8_into<0xC>(a0.x, b0.x), ror8_into<0xC>(a0.y, b0.y), ror8_into<0xC>(a0.z, b0.z),
                  ror8_into<0xC>(a0.w, b0.w));
  b = make_float4(ror8_into<0x3>(b0.x, a0.x), ror8_into<0x3>(b0.y, a0.y), ror8_into<0x3>(b0.z, a0.z),
                  ror8_into<0x3>(b0.w, a0.w));
}

// Row (within the row tile) and column of what lane (r, cq) moves in
// instruction A of a pair; instruction B is eight rows further down.
__device__ __forceinline__ int line_row(int r) { return r & 7; }
__device__ __forceinline__ int line_col(int r, int cq) { return ((r & 8) ? 16 : 0) + cq * 4; }

// Issue the loads of a head's d x n state (wave w: row tiles w * RT ..) in the
// line arrangement; every pair must pass settle_pair before it is used.
template <int N, int RT, int NCT>
__device__ __forceinline__ void load_state_lines(float4 (&s)[RT][NCT], const float* S, int wave, int r, int cq) {
  static_assert(NCT % 2 == 0, "pairs of column tiles");
  // (addresses written as base + row offset + column offset: summing the two
  // offsets first took more registers and made the GDN verify spill)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ra = (wave * RT + rt) * 16 + line_row(r), co = line_col(r, cq);
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      s[rt][2 * jj] = ld_f4_nt(S + ra * N + 32 * jj + co);
      s[rt][2 * jj + 1] = ld_f4_nt(S + (ra + 8) * N + 32 * jj + co);
    }
  }
}

// Every pair of a loaded state into the tile layout.
template <int RT, int NCT>
__device__ __forceinline__ void settle_state(float4 (&s)[RT][NCT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) settle_pair(s[rt][2 * jj], s[rt][2 * jj + 1]);
}

// Store the pair of column tiles 2jj, 2jj + 1 of row tile `rowtile` given in the
// tile layout (a = tile 2jj, b = tile 2jj + 1) as whole lines.
template <int N>
__device__ __forceinline__ void store_pair_lines(float* S, int rowtile, int jj, float4 a, float4 b, int r, int cq) {
  settle_pair(a, b);
  const int ra = rowtile * 16 + line_row(r), co = line_col(r, cq);
  st_f4_nt(S + ra * N + 32 * jj + co, a);
  st_f4_nt(S + (ra + 8) * N + 32 * jj + co, b);
}

__device__ __forceinline__ float dot4_bf16(float4 s, uint2 q) {
  return s.x * bf16_lo(q.x) + s.y * bf16_hi(q.x) + s.z * bf16_lo(q.y) + s.w * bf16_hi(q.y);
}

__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b) {
  return bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
         bf16_hi(a.y) * bf16_hi(b.y) + bf16_lo(a.z) * bf16_lo(b.z) + bf16_hi(a.z) * bf16_hi(b.z) +
         bf16_lo(a.w) * bf16_lo(b.w) + bf16_hi(a.w) * bf16_hi(b.w);
}

__device__ __forceinline__ float dot4_bf16x(uint2 a, uint2 b) {
  return bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
         bf16_hi(a.y) * bf16_hi(b.y);
}

template <typename V> __device__ __forceinline__ V zero_chunk();
template <> __device__ __forceinline__ uint2 zero_chunk<uint2>() { return make_uint2(0, 0); }
template <> __device__ __forceinline__ uint4 zero_chunk<uint4>() { return make_uint4(0, 0, 0, 0); }

// A key or query vector of n bf16 values spread over 16 lanes: lane `sub` holds
// columns sub * n / 16 .. +n/16 as C chunks of W values (n = 64: one 8-byte
// chunk; 128: one 16-byte chunk; 256: two).
template <int N> struct KeyLanes;
template <> struct KeyLanes<64> {
  using Chunk = uint2;
  static constexpr int C = 1, W = 4;
  __device__ static float dot(Chunk a, Chunk b) { return dot4_bf16x(a, b); }
};
template <> struct KeyLanes<128> {
  using Chunk = uint4;
  static constexpr int C = 1, W = 8;
  __device__ static float dot(Chunk a, Chunk b) { return dot8_bf16(a, b); }
};
template <> struct KeyLanes<256> {
  using Chunk = uint4;
  static constexpr int C = 2, W = 8;
  __device__ static float dot(Chunk a, Chunk b) { return dot8_bf16(a, b); }
};

// Per-(request, head) ring record: words 0-1 the pointer word (head in bits
// 0-15, count 16-31, pending 32-47), word 2 the head's A (Mamba-2), word 3 + s
// the step size (Mamba-2) or decay (GDN) of physical slot s.  Each head has its
// own record and every call moves all of a request's records alike, so the work
// of head h reads and writes only record h.
constexpr int kMetaPtr = 0, kMetaA = 2, kMetaSlot = 3;
__host__ __device__ constexpr int meta_words(int L) { return L + kMetaSlot <= 32 ? 32 : 64; }
static_assert(sizeof(rssm_ring_record) == 128 && offsetof(rssm_ring_record, A) == 4 * kMetaA &&
                  offsetof(rssm_ring_record, slot) == 4 * kMetaSlot,
              "record words as the kernels index them");
static_assert(RSSM_META_WORDS(16) == meta_words(16) && RSSM_META_WORDS(32) == meta_words(32),
              "record size as the header states it");
struct RingPtr {
  int head, count, pending;
};

__device__ __forceinline__ RingPtr unpack_ptr(unsigned long long w) {
  return {int(w & 0xFFFFu), int((w >> 16) & 0xFFFFu), int((w >> 32) & 0xFFFFu)};
}

__device__ __forceinline__ unsigned long long pack_ptr(int head, int count, int pending) {
  return (unsigned long long)(head & 0xFFFF) | ((unsigned long long)(count & 0xFFFF) << 16) |
         ((unsigned long long)(pending & 0xFFFF) << 32);
}

__device__ __forceinline__ void flag_error(int32_t* err, int bits) {
  if (err != nullptr && bits != 0) atomicOr(err, bits);
}

// Device-side commit of a draft window: count += clamp(accepted, 0, pending),
// pending = 0; a pending or count out of range is clamped and flagged first.
// Used by the commit kernel and, folded into the next verify, by the
// commit-and-verify calls.
__device__ __forceinline__ void commit_window(int L, int acc, int& cnt, int& pend, int& bad) {
  if (pend > L) {
    pend = L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt + pend > L) {
    cnt = L - pend;
    bad |= RSSM_ERR_POINTERS;
  }
  if (acc < 0 || acc > pend) {
    acc = acc < 0 ? 0 : pend;
    bad |= RSSM_ERR_ACCEPTED;
  }
  cnt += acc;
  pend = 0;
}

// Zero, from v_mbcnt_lo with an empty lane mask (it counts no lanes), which the
// compiler cannot prove equal in every lane.  Added to the index of a load whose
// address is the same for the whole wave, it keeps the load per-lane: the value
// stays in vector registers and is waited for where it is first used.  A uniform
// load is instead copied to a scalar register, and waited for, right after it is
// issued: every work-group of the window kernel waited one memory round trip for
// its ring record before issuing its checkpoint loads (append-decode 2.4 %, the
// fused front-end 4.7 %, a verify round 3 % slower).
__device__ __forceinline__ int opaque_zero() { return (int)__builtin_amdgcn_mbcnt_lo(0u, 0u); }

// Pool row of batch entry b: b itself without a slot map, else slots[b]; -1
// when the entry is skipped (a negative slot marks padding; a slot past the
// pool is also flagged).  Uniform per request.
__device__ __forceinline__ int pool_row(const int32_t* slots, int rows, int b, int32_t* err,
                                        bool report) {
  if (slots == nullptr) return b;
  const int s = slots[b];
  if (s >= rows) {
    if (report) flag_error(err, RSSM_ERR_SLOT);
    return -1;
  }
  return s < 0 ? -1 : s;
}

// One fp32 MFMA step of the transposed tile product: acc[m][nn] += sum_k a[m][k] b[k][nn]
// with lane l supplying a[l & 15][l >> 4] and b[l >> 4][l & 15].
__device__ __forceinline__ v4f mfma4(float a, float b, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Two bf16 MFMA operands whose sum is the fp32 vector x: hi = the upper halves
// (truncation), lo = the remainders x - hi (exact in fp32) cut to bf16.  hi + lo
// is within 2^-14 of x relative; products with bf16 values are exact in the fp32
// accumulator.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ua = __float_as_uint(x[2 * e]), ub = __float_as_uint(x[2 * e + 1]);
    hi[e] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // [ua.hi16 | ub.hi16 << 16]
    const float la = x[2 * e] - __uint_as_float(ua & 0xFFFF0000u);
    const float lb = x[2 * e + 1] - __uint_as_float(ub & 0xFFFF0000u);
    lo[e] = __builtin_amdgcn_perm(__float_as_uint(lb), __float_as_uint(la), 0x07060302u);
  }
}

// Per-lane slice of the entries used in the output combine and the fold: lane
// (r, cq) handles entries j = cq + 4m, m < kMaxL / 4.
constexpr int kVJ = kMaxL / 4;

// Fold F cached entries into the checkpoint tiles held in registers (tile layout)
// and store them as whole lines:
//   S_0 <- fabar S_0 + sum_{j<F} fw_j x_j k_j^T   (x = v for Mamba-2, u for GDN)
// on the matrix cores (transposed tile product, K axis = ring entries).
// sk: keys of entries 0..F-1 in LDS, row-major [j][N] bf16; fw: weights in LDS;
// vj[rt][m] = x_{cq+4m}[row of tile rt] for this lane.
template <int D, int N, int RT, int NCT, int VJ>
__device__ __forceinline__ void fold_and_store(float* S0, float4 (&s)[RT][NCT], float fab,
                                               const uint16_t* sk, const float* fw,
                                               const float (&vj)[RT][VJ], int F, int wave,
                                               int r, int cq) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float bop[VJ];
#pragma unroll
    for (int ks = 0; ks < VJ; ++ks) {
      const int j = 4 * ks + cq;
      bop[ks] = (j < F) ? fw[j] * vj[rt][ks] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      float4 o[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ct = 2 * jj + half;
        v4f acc = {fab * s[rt][ct].x, fab * s[rt][ct].y, fab * s[rt][ct].z, fab * s[rt][ct].w};
#pragma unroll
        for (int ks = 0; ks < VJ; ++ks) {
          if (4 * ks >= F) break;  // uniform across the work-group
          const int j = 4 * ks + cq;
          const float aop = (j < F) ? bf16_to_f32(sk[j * N + ct * 16 + r]) : 0.f;
          acc = mfma4(aop, bop[ks], acc);
        }
        o[half] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      store_pair_lines<N>(S0, wave * RT + rt, jj, o[0], o[1], r, cq);
    }
  }
}

}  // namespace rssm

// ---------------------------------------------------------------- host side
namespace rssm_host {

template <typename P>
inline int launch(void (*kern)(P), dim3 grid, dim3 block, void* stream, const P& params) {
  void* args[] = {const_cast<P*>(&params)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, args, 0,
                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSSM_OK : RSSM_ELAUNCH;
}

inline bool dims_ok(const rssm_dims* d) {
  if (d == nullptr) return false;
  if (d->batch < 1 || d->nheads < 1 || d->ngroups < 1 || d->head_dim < 1 || d->state_dim < 1)
    return false;
  if (d->nheads % d->ngroups != 0) return false;
  if (d->flags & ~(RSSM_F_Y_BF16 | RSSM_F_U_BF16)) return false;
  // one work-group of kBlock threads per (request, head): the grid's work-item
  // count has to fit 32 bits
  if ((long long)d->batch * d->nheads > 0xFFFFFFFFLL / rssm::kBlock) return false;
  return true;
}

// Every decode call, the fused front-end included: head dims d in {64, 128},
// state sizes n in {64, 128, 256}.
inline bool shape_supported(const rssm_dims* d) {
  return (d->head_dim == 64 || d->head_dim == 128) &&
         (d->state_dim == 64 || d->state_dim == 128 || d->state_dim == 256);
}

inline bool ring_shape_supported(const rssm_dims* d) {
  return shape_supported(d) && d->capacity <= rssm::kMaxL;
}

inline bool conv_shape_supported(const rssm_dims* d) { return ring_shape_supported(d); }

// Every array argument is 16-byte aligned (the kernels move 16-byte chunks;
// hipMalloc returns 256-byte aligned memory); null pointers pass here and are
// checked where they are required.
inline bool aligned16() { return true; }
template <typename T, typename... Rest>
inline bool aligned16(const T* p, Rest... rest) {
  return reinterpret_cast<uintptr_t>(p) % 16 == 0 && aligned16(rest...);
}

inline bool meta_ok(const rssm_ring* r) {
  return r != nullptr && r->meta != nullptr && reinterpret_cast<uintptr_t>(r->meta) % 128 == 0 &&
         (r->slots == nullptr || r->rows >= 1) && aligned16(r->slots) &&
         reinterpret_cast<uintptr_t>(r->err) % 4 == 0;
}

inline bool ring_ok(const rssm_ring* r) {
  return meta_ok(r) && r->vu != nullptr && r->k != nullptr && aligned16(r->vu, r->k);
}

}  // namespace rssm_host
