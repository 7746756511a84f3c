// ReplaySSM window kernel (append-decode and T-draft verify) and its launcher,
// shared by the translation units that instantiate it.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- method (core idea,
// output-only decode, rollback as a pointer move), algorithms (Mamba-2 standard
// decode; speculative decoding with the early-flush rule) and kernel design
// (shared inner products, ring indexed in-kernel).
#pragma once

#include "common.hpp"

namespace rssm {

// ======================================================= ReplaySSM
struct ReplayParams {
  float* state0;
  uint16_t* ring_v;
  uint16_t* ring_k;
  float* ring_dt;
  float* ring_decay;
  int32_t* head;
  int32_t* count;
  int32_t* pending;
  int32_t* arrive;
  int32_t* err;
  const uint16_t* v;   // [B, T, H, D]
  const uint16_t* k;   // [B, T, G, N]
  const uint16_t* q;   // [B, T, G, N]
  const float* dt;     // [B, T, H]
  const float* dt_bias;
  const float* A;
  float* y;            // [B, T, H, D]
  int32_t* flushed;
  const int32_t* mask;  // explicit flush only
  int H, G, L;
};

// Load the checkpoint tiles of one head (tile layout) into registers.
template <int D, int N, int RT, int NCT>
__device__ __forceinline__ void load_tiles(float4 (&s)[RT][NCT], const float* S0, int wave, int r,
                                           int cq) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S0 + row * N + ct * 16 + cq * 4);
  }
}

// One kernel for both decode modes.
//  APPEND (T == 1): append the token; it is entry c of E = c + 1; flush all E
//    entries when E == L (flush-when-full).  count <- E or 0.
//  VERIFY (T drafts): drafts are entries c .. c+T-1; draft s reads p_s = c+s+1
//    entries; if c + 2T > L fold the c committed entries only.  pending <- T.
// A work-group serves HPW consecutive heads of one group: the queries, the ring
// keys and the inner products k_j . q_s are shared by them and computed once.  With
// DB the checkpoints of two heads are in flight at a time (two register buffers);
// without it the next head is fetched into the one buffer once it is consumed.  LCAP (16 or 32) bounds L and sizes the per-lane entry
// arrays.  Every global load is issued unconditionally with clamped indices
// (results selected afterwards), so loads go out back to back and the first wait
// comes at the first use.
template <int D, int N, int T, bool APPEND, int LCAP, int HPW, bool DB>
__global__ __launch_bounds__(kBlock) void replay_window_kernel(ReplayParams p) {
  static_assert(N == 128, "key/query staging assumes n = 128 (16 lanes x 8 values)");
  static_assert(LCAP == 16 || LCAP == 32, "ring capacity bound");
  static_assert(HPW >= 1 && HPW <= kWavesPerBlock, "one weight scan per wave");
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  constexpr int VJ = LCAP / 4;         // entries per lane in the combine and fold
  constexpr int PASSES = LCAP / 16;    // inner-product passes of 16 entries
  constexpr int NEWV = T * D / 8;      // 16-byte chunks of one head's new v
  constexpr int NEWK = T * N / 8;      // ... of the group's new k
  constexpr int NCH = HPW * NEWV + NEWK;
  constexpr int NCP = (NCH + kBlock - 1) / kBlock;  // new-entry chunks per thread
  __shared__ float s_w[HPW][T][LCAP];  // w_{j,s} per head, zero where j >= p_s
  __shared__ float s_M[T][LCAP];       // k_j . q_s (shared by the group)
  __shared__ float s_abar[HPW][T];
  __shared__ float s_fw[HPW][LCAP];
  __shared__ float s_fabar[HPW];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[T * N];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[LCAP * N];

  const int H = p.H, G = p.G, L = p.L;
  const int wpr = H / HPW;  // work-groups per request
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / wpr, h0 = (wg - b * wpr) * HPW, hpg = H / G, g = h0 / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4, sub = lane & 15;
  const size_t bh0 = (size_t)b * H + h0;

  // ---- checkpoint tiles of the first two heads: no ring pointer needed
  float4 sa[RT][NCT], sb[RT][NCT];
  load_tiles<D, N, RT, NCT>(sa, p.state0 + bh0 * D * N, wave, r, cq);
  if (DB && HPW > 1) load_tiles<D, N, RT, NCT>(sb, p.state0 + (bh0 + 1) * D * N, wave, r, cq);
  // queries (8 columns per lane) and the new entries' v / k, all pointer-free
  uint4 qm[T];
#pragma unroll
  for (int sd = 0; sd < T; ++sd) qm[sd] = ld_u4(p.q + (((size_t)b * T + sd) * G + g) * N + sub * 8);
  const bool k_owner = (h0 % hpg) == 0;
  // chunk t < HPW*NEWV: v of head h0 + t / NEWV; then NEWK chunks of the group's k
  uint4 newc[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int t = min(tid + i * kBlock, NCH - 1);
    const uint16_t* src;
    if (t < HPW * NEWV) {
      const int hh = t / NEWV, tv = t - hh * NEWV;
      src = p.v + (((size_t)b * T + tv / (D / 8)) * H + h0 + hh) * D + (tv % (D / 8)) * 8;
    } else {
      const int tk = t - HPW * NEWV;
      src = p.k + (((size_t)b * T + tk / (N / 8)) * G + g) * N + (tk % (N / 8)) * 8;
    }
    newc[i] = ld_u4(src);
  }

  // ---- ring pointers (uniform per request), clamped into range
  int head = p.head[b], cnt = p.count[b];
  const int pend = p.pending[b];
  int bad = 0;
  if (head < 0 || head >= L) {
    head = ((head % L) + L) % L;
    bad |= RSSM_ERR_POINTERS;
  }
  const int cmax = APPEND ? L - 1 : L - T;
  if (cnt < 0 || cnt > cmax) {
    cnt = cnt < 0 ? 0 : cmax;
    bad |= RSSM_ERR_POINTERS;
  }
  if (pend != 0) bad |= RSSM_ERR_PENDING;
  const int c = cnt;
  const int E = c + T;
  const bool do_flush = APPEND ? (E == L) : (c + 2 * T > L);
  const int F = do_flush ? (APPEND ? E : c) : 0;
  const bool write_new = !(APPEND && do_flush);
  int arrival = 0;
  if (tid == 0) arrival = arrive_after_reading(&p.arrive[b], head, cnt, pend);

  // ---- v_j[row] of the first two heads for the entries this lane combines
  //      (j = cq + 4m); later heads are fetched with their checkpoint tiles
  float va[RT][VJ], vb[RT][VJ];
  auto load_v = [&](float (&vj)[RT][VJ], int i) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
      for (int m = 0; m < VJ; ++m) {
        const int j = cq + 4 * m;
        const int jj = min(j, E - 1);
        const uint16_t* src = (jj < c) ? p.ring_v + ((bh0 + i) * L + ring_slot(head, jj, L)) * D
                                       : p.v + (((size_t)b * T + max(jj - c, 0)) * H + h0 + i) * D;
        const float val = bf16_to_f32(src[row]);
        vj[rt][m] = (j < E) ? val : 0.f;
      }
    }
  };
  load_v(va, 0);
  if (DB && HPW > 1) load_v(vb, 1);
  // ---- keys of the entries for the shared inner products (16 lanes per entry)
  uint4 kj[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = ps * 16 + wave * 4 + (lane >> 4);
    const int jj = min(j, E - 1);
    const uint16_t* src = (jj < c)
        ? p.ring_k + (((size_t)b * G + g) * L + ring_slot(head, jj, L)) * N
        : p.k + (((size_t)b * T + max(jj - c, 0)) * G + g) * N;
    kj[ps] = ld_u4(src + sub * 8);
  }

  // ---- wave i: step sizes and decays of head h0+i, then its weights by
  //      suffix-product scans (one per draft boundary, one for the fold)
  if (wave < HPW) {
    const int i = wave, hh = h0 + wave;
    const size_t bh = bh0 + i;
    const int j = lane;
    const int jj = min(j, E - 1);
    const size_t o = bh * L + ring_slot(head, max(min(jj, c - 1), 0), L);
    const float dl_ring = p.ring_dt[o], al_ring = p.ring_decay[o];
    const int sdj = max(jj - c, 0);
    const float dl_new = softplus_f32(p.dt[((size_t)b * T + sdj) * H + hh] + p.dt_bias[hh]);
    const float al_new = expf(p.A[hh] * dl_new);
    const bool valid = j < E, cached = jj < c;
    const float dl = valid ? (cached ? dl_ring : dl_new) : 0.f;
    const float al = valid ? (cached ? al_ring : al_new) : 1.f;
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const int m = c + sd;  // last entry seen by draft sd
      float all;
      const float ex = suffix_product_excl(j <= m ? al : 1.f, lane, &all);
      if (j < LCAP) s_w[i][sd][j] = (j <= m) ? dl * ex : 0.f;
      if (lane == 0) s_abar[i][sd] = all;
    }
    {
      float all;
      const float ex = suffix_product_excl(j < F ? al : 1.f, lane, &all);
      if (j < LCAP) s_fw[i][j] = (j < F) ? dl * ex : 0.f;
      if (lane == 0) s_fabar[i] = all;
    }
    if (write_new && j >= c && j < E) {  // cache the new entries' step size and decay
      const size_t on = bh * L + ring_slot(head, j, L);
      p.ring_dt[on] = dl;
      p.ring_decay[on] = al;
    }
  }
  if (wave == 0 && lane < 16) {
#pragma unroll
    for (int sd = 0; sd < T; ++sd) *reinterpret_cast<uint4*>(&s_q[sd * N + sub * 8]) = qm[sd];
  }

  // ---- all waves: inner products and staging of the keys to fold
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = ps * 16 + wave * 4 + (lane >> 4);
    const uint4 kv = (j < E) ? kj[ps] : make_uint4(0, 0, 0, 0);
    if (j < F) *reinterpret_cast<uint4*>(&s_k[j * N + sub * 8]) = kv;
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const float dv = reduce_quarter(dot8_bf16(kv, qm[sd]));
      if (sub == 0) s_M[sd][j] = dv;
    }
  }
  __syncthreads();

  // ---- per head: output-only route y_s = abar_s (S_0 q_s) + sum_j w_{j,s} M_{j,s} v_j,
  //      then the fold when flushing; the next-but-one head is loaded into the
  //      buffer just consumed
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    float4 (&s)[RT][NCT] = (DB && (i & 1)) ? sb : sa;
    float (&vj)[RT][VJ] = (DB && (i & 1)) ? vb : va;
    const size_t bh = bh0 + i;
    float* S0 = p.state0 + bh * D * N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
      float dots[T];
#pragma unroll
      for (int sd = 0; sd < T; ++sd) dots[sd] = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int sd = 0; sd < T; ++sd)
          dots[sd] += dot4_bf16(s[rt][ct], *reinterpret_cast<const uint2*>(&s_q[sd * N + ct * 16 + cq * 4]));
#pragma unroll
      for (int sd = 0; sd < T; ++sd) {
        float part = s_abar[i][sd] * dots[sd];
#pragma unroll
        for (int m = 0; m < VJ; ++m) {
          const int j = cq + 4 * m;
          part += s_w[i][sd][j] * s_M[sd][j] * vj[rt][m];  // both zero beyond p_s
        }
        part = reduce_row4(part);
        if ((sd & 3) == cq) p.y[(((size_t)b * T + sd) * H + h0 + i) * D + row] = part;
      }
    }
    if (F > 0)
      fold_and_store<D, N, RT, NCT, VJ>(S0, s, s_fabar[i], s_k, s_fw[i], vj, F, wave, r, cq);
    constexpr int ahead = DB ? 2 : 1;  // the buffer just consumed takes head i + ahead
    if (i + ahead < HPW) {
      load_tiles<D, N, RT, NCT>(s, p.state0 + (bh + ahead) * D * N, wave, r, cq);
      load_v(vj, i + ahead);
    }
  }

  // ---- cache the new entries' v (every head here) and k (group owner only)
  if (write_new) {
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int t = tid + i * kBlock;
      if (t < HPW * NEWV) {
        const int hh = t / NEWV, tv = t - hh * NEWV;
        const int sd = tv / (D / 8), o = (tv % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(p.ring_v + ((bh0 + hh) * L + ring_slot(head, c + sd, L)) * D + o) = newc[i];
      } else if (k_owner && t < NCH) {
        const int tk = t - HPW * NEWV;
        const int sd = tk / (N / 8), o = (tk % (N / 8)) * 8;
        *reinterpret_cast<uint4*>(p.ring_k + (((size_t)b * G + g) * L + ring_slot(head, c + sd, L)) * N + o) = newc[i];
      }
    }
  }

  // ---- pointer update by the last work-group of the request to read them
  if (tid == 0) {
    if (h0 == 0) {
      flag_error(p.err, bad);
      if (p.flushed != nullptr) p.flushed[b] = do_flush ? 1 : 0;
    }
    if (arrival == wpr - 1) {
      p.arrive[b] = 0;
      if (APPEND) {
        p.head[b] = do_flush ? ring_slot(head, E % L, L) : head;
        p.count[b] = do_flush ? 0 : E;
        p.pending[b] = 0;
      } else {
        p.head[b] = do_flush ? ring_slot(head, c % L, L) : head;
        p.count[b] = do_flush ? 0 : c;
        p.pending[b] = T;
      }
    }
  }
}

}  // namespace rssm

namespace rssm_host {

using rssm::ReplayParams;

// Work-group shape: heads per work-group and double buffering.  Four heads with two
// state buffers in flight when the group size allows it (measured best on the
// 32-head, 8-group layer; 1, 2 or 4 heads with one or two buffers all stream within
// 3% of each other there), else one head per work-group.
struct WindowShape {
  int hpw;
  bool db;
};

inline WindowShape window_shape(const ReplayParams& p) {
  const int hpg = p.H / p.G;
  if (hpg % 4 == 0) return {4, true};
  return {1, false};
}

template <int D, int T, bool APPEND, int LCAP>
int launch_window_cap(const ReplayParams& p, WindowShape sh, int B, void* stream) {
  const dim3 grid(B * (p.H / sh.hpw)), block(rssm::kBlock);
  if (sh.hpw == 4) return launch(rssm::replay_window_kernel<D, 128, T, APPEND, LCAP, 4, true>, grid, block, stream, p);
  return launch(rssm::replay_window_kernel<D, 128, T, APPEND, LCAP, 1, false>, grid, block, stream, p);
}

template <int D, int T, bool APPEND>
int launch_window(const ReplayParams& p, int B, void* stream) {
  const WindowShape sh = window_shape(p);
  if (p.L <= 16) return launch_window_cap<D, T, APPEND, 16>(p, sh, B, stream);
  return launch_window_cap<D, T, APPEND, 32>(p, sh, B, stream);
}

// Verify launchers for T = 1..4 and T = 5..8 live in their own translation units.
__attribute__((visibility("hidden"))) int launch_replay_verify_lo(int T, int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_verify_hi(int T, int D, const ReplayParams& p, int B, void* stream);

}  // namespace rssm_host
