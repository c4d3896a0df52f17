// Device routines of the routing step: top-k selection of one token and the
// token -> expert route tables, for one 256-thread workgroup.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega (sigmoid scoring with one group,
// normalised top-k weights times routed_scaling_factor) and
// LayerStages._mega_moe (the score-correction bias goes with the logits; the
// boundary receives the route order with the unfinalized rows).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kRouteThreads = 256;

// A logit as stored by the router: plain fp32, or (ENC) its bits inverted,
// so that zeroed memory reads as "not written yet" (inverted bits of 0 are a
// NaN pattern no dot product produces) and a consumer can poll the logits
// themselves instead of a counter.
template <bool C, bool ENC>
__device__ __forceinline__ float load_logit(const float* p) {
  const float v = ld_f32<C>(p);
  return ENC ? __uint_as_float(~__float_as_uint(v)) : v;
}

// Polls before a wait for logits gives up (a poll is a memory round trip
// plus a short sleep; a legitimate wait lasts microseconds).
constexpr uint32_t kLogitPolls = 1u << 17;

// Lane l's logits of experts l + 64 i (i < N) of one token into sc (clamped
// index past E).  POLL (encoded logits only): the wave repeats the loads
// until every logit of the token has been stored (none reads 0); after
// kLogitPolls rounds it sets *err and goes on.  Then ENC decodes them.
template <bool C, bool ENC, bool POLL, int N>
__device__ __forceinline__ void load_token_logits(const float* logits, int E, float* sc,
                                                  uint32_t* err) {
  static_assert(!POLL || ENC, "only encoded logits can be polled");
  const int lane = threadIdx.x & 63;
  uint32_t polls = 0;
  for (;;) {
    bool have = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = lane + 64 * i;
      sc[i] = ld_f32<C>(logits + (e < E ? e : E - 1));
      have = have && (e >= E || __float_as_uint(sc[i]) != 0u);
    }
    if (!POLL || __builtin_amdgcn_ballot_w64(!have) == 0) break;  // uniform
    if (++polls == kLogitPolls) {
      if (lane == 0)
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (ENC) {
#pragma unroll
    for (int i = 0; i < N; ++i) sc[i] = __uint_as_float(~__float_as_uint(sc[i]));
  }
}

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of v over the wave with DPP moves: shifts by 1, 2, 4, 8
// within rows of 16 lanes (lanes with no source add 0), then the last lane of
// row 0 is added to row 1 and of row 2 to row 3 (row_bcast:15), and the last
// lane of row 1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive scan of v over the 256 threads (4 waves); returns the prefix and
// writes the total to *total.  s_tmp holds 4 ints.
__device__ inline int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = s_tmp[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Per-wave LDS scratch of select_token, in 8-byte words: the 64 lane
// maxima, the candidate keys (kMaxTopK lanes x 16 slots, plus zero padding
// to a multiple of 8), the picks and the threshold (padded to a 16-byte
// multiple).
constexpr int kSelWaveWords = (64 + kMaxTopK * 16 + 8 + kMaxTopK + 1 + 1) & ~1;
constexpr size_t kSelBytes = static_cast<size_t>(kRouteThreads / 64) * kSelWaveWords * 8;

// Orders the LDS accesses of one wave: the compiler keeps them on their side
// of this point, and a wave's LDS instructions complete in issue order, so
// what every lane wrote before it is what every lane reads after it.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Top-k of one token in one wave.  Keys are sigmoid(logit) + bias (bias is
// never null: a zero vector stands in for no bias); the largest key wins,
// equal keys go to the lower expert id.  Lane l holds experts l + 64 i
// (slot i < ceil(E / 64)) as unique 64-bit keys (order-preserving key bits,
// then ~id; 0 for a slot past E).
//
// Selection without serial rounds: tau = the k-th largest of the 64 lane
// maxima (each lane counts the lane maxima above its own).  The k lanes
// whose maximum reaches tau hold k keys >= tau, so every top-k key is
// >= tau, and a key >= tau can only sit in one of those lanes.  They write
// their keys >= tau to LDS (a k x ceil(E / 64) table, other entries 0), and
// every candidate's rank is the number of table entries above it: every key
// above a candidate is itself a candidate.  Rank j < k is the j-th pick.
// A few LDS round trips replace k rounds of wave arg-max, each of which
// waits on vector-to-scalar dependencies.  Lane j < k ends with the j-th
// pick and its weight R * s_j / (s_0 + ... + s_{k-1}), summed in pick
// order.  sel: this wave's kSelWaveWords words of LDS.
//
// NS = slots per lane, a power of two >= ceil(E / 64) (slots past E hold
// key 0), so that every loop over a lane's keys unrolls with constant
// indices.
template <bool C, int NS, bool ENC = false, bool POLL = false>
__device__ inline void select_token_ns(const float* logits, const float* bias, int E, int k,
                                       float rsf, unsigned long long* sel, int* pick_id,
                                       float* pick_w, uint32_t* err = nullptr) {
  const int lane = threadIdx.x & 63;
  unsigned long long* lmax = sel;
  unsigned long long* cand = sel + 64;
  unsigned long long* picks = cand + kMaxTopK * 16 + 8;
  unsigned long long* thr = picks + kMaxTopK;
  float sc[NS];
  float bv[NS];
  unsigned long long key[NS];
  // every load first (clamped index)
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    bv[i] = bias[e < E ? e : E - 1];
  }
  load_token_logits<C, ENC, POLL, NS>(logits, E, sc, err);
  unsigned long long mx = 0ull;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    const float s = sigmoidf_(sc[i]);
    sc[i] = s;
    key[i] = e < E ? (static_cast<unsigned long long>(ordered_bits(s + bv[i])) << 32) |
                         (0xffffffffu - static_cast<uint32_t>(e))
                   : 0ull;
    mx = key[i] > mx ? key[i] : mx;
  }
  lmax[lane] = mx;
  wave_lds_order();
  // lane maxima above this lane's: 16 keys per batch, the batch's loads first
  int rank = 0;
#pragma unroll
  for (int j0 = 0; j0 < 64; j0 += 16) {
    ulonglong2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = reinterpret_cast<const ulonglong2*>(lmax + j0)[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) rank += (v[j].x > mx ? 1 : 0) + (v[j].y > mx ? 1 : 0);
  }
  if (rank == k - 1) *thr = mx;
  wave_lds_order();
  const unsigned long long tau = *thr;
  const bool holds = rank < k;  // exactly k lanes
  if (holds) {
#pragma unroll
    for (int i = 0; i < NS; ++i) cand[rank * NS + i] = key[i] >= tau ? key[i] : 0ull;
  }
  // the table is padded with zeros to a multiple of 8 entries
  const int nc = k * NS, nc8 = (nc + 7) & ~7;
  if (lane < nc8 - nc) cand[nc + lane] = 0ull;
  wave_lds_order();
  if (holds) {
    int r[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) r[i] = 0;
    for (int j0 = 0; j0 < nc8; j0 += 8) {
      ulonglong2 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = reinterpret_cast<const ulonglong2*>(cand + j0)[j];
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r[i] += (v[j].x > key[i] ? 1 : 0) + (v[j].y > key[i] ? 1 : 0);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (key[i] >= tau && r[i] < k)
        picks[r[i]] = (static_cast<unsigned long long>(__float_as_uint(sc[i])) << 32) |
                      static_cast<uint32_t>(lane + 64 * i);
  }
  wave_lds_order();
  if (lane < k) {
    const unsigned long long p = picks[lane];
    float ssum = 0.f;
    for (int j = 0; j < k; ++j) ssum += __uint_as_float(static_cast<uint32_t>(picks[j] >> 32));
    *pick_id = static_cast<int>(static_cast<uint32_t>(p));
    *pick_w = rsf * __uint_as_float(static_cast<uint32_t>(p >> 32)) / ssum;
  }
  wave_lds_order();  // the next token's writes come after these reads
}

// One step of the DPP wave maximum of 64-bit values held as (hi, lo)
// dwords: lanes take the neighbour's value named by the DPP control when it
// is larger (one 64-bit compare).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t h2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, BANK_MASK, false);
  const uint32_t l2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, BANK_MASK, false);
  const unsigned long long a = (static_cast<unsigned long long>(hi) << 32) | lo;
  const unsigned long long b = (static_cast<unsigned long long>(h2) << 32) | l2;
  const bool take = b > a;
  hi = take ? h2 : hi;
  lo = take ? l2 : lo;
}

// Maximum of the (hi, lo) pairs of the 64 lanes, lexicographic, in every
// lane: shifts within rows of 16 lanes, then row broadcasts 15 and 31 carry
// the rows' maxima up to lane 63, which is read back to all lanes.
__device__ __forceinline__ void wave_max_pair(uint32_t& hi, uint32_t& lo) {
  dpp_max_step<0x111, 0xf, 0xf>(hi, lo);  // row_shr:1
  dpp_max_step<0x112, 0xf, 0xf>(hi, lo);  // row_shr:2
  dpp_max_step<0x113, 0xf, 0xf>(hi, lo);  // row_shr:3
  dpp_max_step<0x114, 0xf, 0xe>(hi, lo);  // row_shr:4
  dpp_max_step<0x118, 0xf, 0xc>(hi, lo);  // row_shr:8
  dpp_max_step<0x142, 0xa, 0xf>(hi, lo);  // row_bcast:15
  dpp_max_step<0x143, 0xc, 0xf>(hi, lo);  // row_bcast:31
  hi = __builtin_amdgcn_readlane(hi, 63);
  lo = __builtin_amdgcn_readlane(lo, 63);
}

// The same selection in k rounds, for more than 256 experts (where the
// threshold table would need more registers than the router kernel can
// spare).  Keys as above, 32-bit order-preserving bits per slot, 0 marking a
// slot that is taken or past E (a real key never maps to 0).  Each round
// takes every lane's best slot (strict >, so the lower slot, i.e. the lower
// id, wins a tie), then a DPP wave maximum of (key, ~id).
template <bool C, bool ENC = false, bool POLL = false>
__device__ inline void select_token_rounds(const float* logits, const float* bias, int E, int k,
                                    float rsf, int* pick_id, float* pick_w,
                                    uint32_t* err = nullptr) {
  const int lane = threadIdx.x & 63;
  const int ns = (E + 63) >> 6;
  float sc[16];
  uint32_t kb[16];
  // Branch-free loads (clamped index).
  float bv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    bv[i] = bias[e < E ? e : E - 1];
  }
  load_token_logits<C, ENC, POLL, 16>(logits, E, sc, err);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const float s = sigmoidf_(sc[i]);
    sc[i] = s;
    kb[i] = e < E ? ordered_bits(s + bv[i]) : 0u;
  }
  float ssum = 0.f, my_s = 0.f;
  int my_id = -1;
  for (int j = 0; j < k; ++j) {
    uint32_t bk = kb[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      if (i >= ns) break;  // uniform
      const bool take = kb[i] > bk;
      bk = take ? kb[i] : bk;
      bi = take ? i : bi;
    }
    uint32_t hi = bk;
    uint32_t lo = bk ? 0xffffffffu - static_cast<uint32_t>(lane + 64 * bi) : 0u;
    wave_max_pair(hi, lo);
    const int win = static_cast<int>(0xffffffffu - lo);
    const int wslot = win >> 6, wlane = win & 63;  // uniform
    float v = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      if (i >= ns) break;
      v = i == wslot ? sc[i] : v;
    }
    const float wsc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), wlane));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i >= ns) break;
      kb[i] = (i == wslot && lane == wlane) ? 0u : kb[i];
    }
    ssum += wsc;
    if (lane == j) {
      my_id = win;
      my_s = wsc;
    }
  }
  if (lane < k) {
    *pick_id = my_id;
    *pick_w = rsf * my_s / ssum;
  }
}

// WIDE = false leaves out the path for more than 256 experts (its sixteen
// keys and scores per lane raise a kernel's register count; a caller that
// sets it must not pass E > 256).
template <bool C, bool ENC = false, bool POLL = false, bool WIDE = true>
__device__ inline void select_token(const float* logits, const float* bias, int E, int k,
                                    float rsf, unsigned long long* sel, int* pick_id,
                                    float* pick_w, uint32_t* err = nullptr) {
  const int ns = (E + 63) >> 6;  // uniform
  if (ns <= 1)
    select_token_ns<C, 1, ENC, POLL>(logits, bias, E, k, rsf, sel, pick_id, pick_w, err);
  else if (ns <= 2)
    select_token_ns<C, 2, ENC, POLL>(logits, bias, E, k, rsf, sel, pick_id, pick_w, err);
  else if (!WIDE || ns <= 4)
    select_token_ns<C, 4, ENC, POLL>(logits, bias, E, k, rsf, sel, pick_id, pick_w, err);
  else
    select_token_rounds<C, ENC, POLL>(logits, bias, E, k, rsf, pick_id, pick_w, err);
}

// LDS bytes select_and_route needs (16-byte aligned base).
__host__ __device__ inline size_t route_smem_bytes(int T, int E, int k) {
  const size_t R = static_cast<size_t>(T) * k, MW = (T + 63) / 64;
  return kSelBytes + ((R * 4 + 7) & ~static_cast<size_t>(7)) +
         static_cast<size_t>(E) * MW * 8 + static_cast<size_t>(E) * 8 + 16;
}

// LDS carve-up of the routing step: the selection scratch of each wave
// [4 * kSelWaveWords], s_ids [T*k], token masks [E * MW], offsets [E],
// touched slot of each expert [E], scan scratch [4].
struct RouteSmem {
  unsigned long long* sel;
  int* ids;
  unsigned long long* mask;
  int* off;
  int* slot;
  int* tmp;
  __device__ RouteSmem(unsigned char* smem, int T, int E, int k) {
    const size_t R = static_cast<size_t>(T) * k, MW = (T + 63) / 64;
    sel = reinterpret_cast<unsigned long long*>(smem);
    smem += kSelBytes;
    ids = reinterpret_cast<int*>(smem);
    mask = reinterpret_cast<unsigned long long*>(smem + ((R * 4 + 7) & ~static_cast<size_t>(7)));
    off = reinterpret_cast<int*>(mask + static_cast<size_t>(E) * MW);
    slot = off + E;
    tmp = slot + E;
  }
};

// Top-k of tokens [t_begin, t_end), one wave per token.  Writes ws.ids and
// ws.weights (coherent stores when C), the optional caller outputs and the
// LDS copy of the ids (route r = t*k + j).
template <bool C, bool ENC = false, bool POLL = false, bool WIDE = true>
__device__ inline void select_tokens(int t_begin, int t_end, int E, int k, float rsf,
                                     const float* logits, const float* bias, const Workspace& ws,
                                     int32_t* ids_out, float* w_out, const RouteSmem& sm,
                                     uint32_t* err = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int* s_ids = sm.ids;
  unsigned long long* sel = sm.sel + static_cast<size_t>(wave) * kSelWaveWords;
  for (int t = t_begin + wave; t < t_end; t += kRouteThreads / 64) {
    int id = 0;
    float w = 0.f;
    select_token<C, ENC, POLL, WIDE>(logits + static_cast<size_t>(t) * E, bias, E, k, rsf, sel,
                                     &id, &w, err);
    if (lane < k) {
      const int r = t * k + lane;
      s_ids[r] = id;
      st_i32<C>(ws.ids + r, id);
      st_f32<C>(ws.weights + r, w);
      if (ids_out) ids_out[r] = id;
      if (w_out) w_out[r] = w;
    }
  }
}

// Route tables of T tokens from the ids in LDS (sm.ids, all T*k routes), by
// one 256-thread workgroup: ws.counts/offsets/touched/n_touched/perm/inv and
// the slot records ws.slot_tab (expert -1 for slots past the touched count,
// up to min(T*k, E)) (coherent stores when C).  Its first barrier comes before the first read of
// sm.ids, so callers may fill sm.ids right before the call.
// One token: its k picks are k distinct experts, one route each.  Expert e's
// position is the number of picks with a lower id; every table follows from
// that without the token masks and the block scan (same tables as below).
template <bool C>
__device__ inline void build_routes_one_token(int E, int k, const Workspace& ws,
                                              const RouteSmem& sm) {
  __syncthreads();  // sm.ids complete
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int below = 0, j_of = -1;
    for (int j = 0; j < k; ++j) {
      const int id = sm.ids[j];
      below += id < e ? 1 : 0;
      j_of = id == e ? j : j_of;
    }
    st_i32<C>(ws.counts + e, j_of >= 0 ? 1 : 0);
    st_i32<C>(ws.offsets + e, below);
    if (j_of >= 0) {
      st_i32<C>(ws.touched + below, e);
      st_i32<C>(ws.perm + below, j_of);
      st_i32<C>(ws.inv + j_of, below);
      int32_t* rec = ws.slot_tab + static_cast<size_t>(below) * kSlotInts;
      st_i32<C>(rec, e);
      st_i32<C>(rec + 1, 1);
      st_i32<C>(rec + 2, below);
      st_i32<C>(rec + 4, j_of);
    }
  }
  if (threadIdx.x == 0) {
    st_i32<C>(ws.offsets + E, k);
    st_i32<C>(ws.n_touched, k);
  }
}

template <bool C>
__device__ inline void build_routes(int T, int E, int k, const Workspace& ws,
                                    const RouteSmem& sm) {
  if (T == 1) {
    build_routes_one_token<C>(E, k, ws, sm);
    return;
  }
  const int R = T * k;
  const int MW = (T + 63) / 64;
  for (int i = threadIdx.x; i < E * MW; i += kRouteThreads) sm.mask[i] = 0ull;
  __syncthreads();

  // Token bitmask of every expert.
  for (int r = threadIdx.x; r < R; r += kRouteThreads) {
    const int e = sm.ids[r], t = r / k;
    atomicOr(&sm.mask[static_cast<size_t>(e) * MW + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  // Counts and touched flags, packed so that one scan gives both prefixes:
  // bits [11, 32) count routes (<= 4096), bits [0, 11) touched experts
  // (<= 1024).  Thread i owns experts 4i .. 4i+3 (E <= 1024).
  {
    int packed[4], local = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = 4 * threadIdx.x + m;
      int cnt = 0;
      if (e < E)
        for (int w = 0; w < MW; ++w) cnt += __popcll(sm.mask[static_cast<size_t>(e) * MW + w]);
      packed[m] = (cnt << 11) | (cnt > 0 ? 1 : 0);
      local += packed[m];
    }
    int total = 0;
    int run = block_exclusive_scan(local, sm.tmp, &total);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = 4 * threadIdx.x + m;
      if (e < E) {
        const int cnt = packed[m] >> 11;
        const int off = run >> 11, tidx = run & 0x7ff;
        sm.off[e] = off;
        sm.slot[e] = tidx;
        st_i32<C>(ws.counts + e, cnt);
        st_i32<C>(ws.offsets + e, off);
        if (cnt > 0) {
          st_i32<C>(ws.touched + tidx, e);
          int32_t* rec = ws.slot_tab + static_cast<size_t>(tidx) * kSlotInts;
          st_i32<C>(rec, e);
          st_i32<C>(rec + 1, cnt);
          st_i32<C>(rec + 2, off);
        }
      }
      run += packed[m];
    }
    if (threadIdx.x == 0) {
      st_i32<C>(ws.offsets + E, total >> 11);
      st_i32<C>(ws.n_touched, total & 0x7ff);
    }
    const int dmax = R < E ? R : E;
    for (int d = (total & 0x7ff) + static_cast<int>(threadIdx.x); d < dmax; d += kRouteThreads)
      st_i32<C>(ws.slot_tab + static_cast<size_t>(d) * kSlotInts, -1);
  }
  __syncthreads();
  // Stable position of every route: its expert's offset plus the number of
  // earlier tokens routed to the same expert.
  for (int r = threadIdx.x; r < R; r += kRouteThreads) {
    const int e = sm.ids[r], t = r / k;
    const unsigned long long* m = sm.mask + static_cast<size_t>(e) * MW;
    int rank = 0;
    for (int w = 0; w < (t >> 6); ++w) rank += __popcll(m[w]);
    rank += __popcll(m[t >> 6] & ((1ull << (t & 63)) - 1ull));
    const int pos = sm.off[e] + rank;
    st_i32<C>(ws.perm + pos, r);
    st_i32<C>(ws.inv + r, pos);
    if (rank < kSlotRoutes)
      st_i32<C>(ws.slot_tab + static_cast<size_t>(sm.slot[e]) * kSlotInts + 4 + rank, r);
  }
}

// Top-k of every token, then the route tables, by one 256-thread workgroup.
// logits [T, E] must be visible to the workgroup.  smem:
// route_smem_bytes(T, E, k) bytes, 16-byte aligned.
template <bool C = false>
__device__ inline void select_and_route(int T, int E, int k, float rsf, const float* logits,
                                        const float* bias, const Workspace& ws,
                                        int32_t* ids_out, float* w_out, unsigned char* smem) {
  const RouteSmem sm(smem, T, E, k);
  select_tokens<C>(0, T, E, k, rsf, logits, bias, ws, ids_out, w_out, sm);
  build_routes<C>(T, E, k, ws, sm);
}

}  // namespace moe
