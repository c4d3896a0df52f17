// Router of the MoE decode layer on gfx950: logits GEMV, sigmoid scores,
// top-k selection with renormalised weights and the token -> expert route
// tables, in one launch.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._router (bf16 router weight, fp32 logits),
// LayerStages._build_mega (sigmoid scoring, one group, normalised top-k,
// routed_scaling_factor) and LayerStages._mega_moe (the route order table
// handed to the boundary with the unfinalized rows).
//
// Phase 1 (every workgroup): each wave computes the logits of kEpw experts
// for a block of kTokB tokens, streaming 16-byte chunks of the bf16 router
// rows; lanes split the hidden dimension and a wave reduction finishes each
// dot product.  Phase 2 (the last workgroup to finish, found with an atomic
// counter): per token a wave ranks the experts with a packed (key, id)
// wave-max, k rounds; then the route tables are built from per-expert token
// bitmasks in LDS (popcounts give stable ranks, one block scan gives the
// offsets and the touched-expert list).  The counter is reset at the end so
// the launch can be replayed from a HIP graph.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kEpw = 2;   // experts per wave
constexpr int kTokB = 8;  // tokens per workgroup row of the grid

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of v over the 256 threads (4 waves); returns the prefix and
// writes the total to *total.  s_tmp holds 4 ints.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int x = s_tmp[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Top-k of one token in one wave.  Keys are sigmoid(logit) (+ bias); equal
// keys go to the lower expert id.  Lane j < k ends with the j-th pick.
__device__ void select_token(const float* logits, const float* bias, int E, int k, float rsf,
                             int* pick_id, float* pick_w) {
  const int lane = threadIdx.x & 63;
  float key[16], sc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int e = lane + 64 * i;
    if (e < E) {
      float s = sigmoidf_(logits[e]);
      sc[i] = s;
      key[i] = bias ? s + bias[e] : s;
    } else {
      sc[i] = 0.f;
      key[i] = 0.f;
    }
  }
  uint32_t taken = 0;
  float ssum = 0.f, my_s = 0.f;
  int my_id = -1;
  for (int j = 0; j < k; ++j) {
    // This lane's best untaken expert (ascending ids, strict > keeps the lower).
    uint32_t bk = 0, bid = 0;
    float bs = 0.f;
    bool have = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int e = lane + 64 * i;
      bool ok = e < E && !((taken >> i) & 1u);
      uint32_t ok_key = ordered_bits(key[i]);
      if (ok && (!have || ok_key > bk)) {
        have = true;
        bk = ok_key;
        bid = static_cast<uint32_t>(e);
        bs = sc[i];
      }
    }
    uint32_t hi = have ? bk : 0u;
    uint32_t lo = have ? (0xffffffffu - bid) : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      uint32_t h2 = __shfl_xor(hi, off, 64), l2 = __shfl_xor(lo, off, 64);
      if (h2 > hi || (h2 == hi && l2 > lo)) {
        hi = h2;
        lo = l2;
      }
    }
    int win = static_cast<int>(0xffffffffu - lo);
    float ws = __shfl(bs, win & 63, 64);
    if (lane == (win & 63)) taken |= 1u << (win >> 6);
    ssum += ws;
    if (lane == j) {
      my_id = win;
      my_s = ws;
    }
  }
  if (lane < k) {
    *pick_id = my_id;
    *pick_w = rsf * my_s / ssum;
  }
}

__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int H, int E, int k, float rsf, Workspace ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, uint32_t total_blocks) {
  // 16-byte aligned: the 64-bit token masks below need 8-byte aligned LDS
  // addresses, and dynamic LDS starts right after the static variables.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  __shared__ int s_tmp[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- phase 1: logits[t, e] for this block's experts and tokens
  {
    const int e0 = (blockIdx.x * 4 + wave) * kEpw;
    const int t0 = blockIdx.y * kTokB;
    const int nt = min(kTokB, T - t0);
    const int nchunk = H / 8;  // 16-byte chunks of a bf16 row
    float acc[kEpw][kTokB];
#pragma unroll
    for (int x = 0; x < kEpw; ++x)
#pragma unroll
      for (int q = 0; q < kTokB; ++q) acc[x][q] = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      float wf[kEpw][8];
#pragma unroll
      for (int x = 0; x < kEpw; ++x) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (e0 + x < E)
          v = *reinterpret_cast<const uint4*>(router_w + static_cast<size_t>(e0 + x) * H + 8 * c);
        uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          wf[x][2 * m] = bf16_lo(u[m]);
          wf[x][2 * m + 1] = bf16_hi(u[m]);
        }
      }
#pragma unroll
      for (int q = 0; q < kTokB; ++q) {
        if (q < nt) {
          uint4 v = *reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(t0 + q) * H + 8 * c);
          uint32_t u[4] = {v.x, v.y, v.z, v.w};
          float xf[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            xf[2 * m] = bf16_lo(u[m]);
            xf[2 * m + 1] = bf16_hi(u[m]);
          }
#pragma unroll
          for (int x = 0; x < kEpw; ++x)
#pragma unroll
            for (int m = 0; m < 8; ++m) acc[x][q] = fmaf(wf[x][m], xf[m], acc[x][q]);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < kEpw; ++x)
#pragma unroll
      for (int q = 0; q < kTokB; ++q) {
        if (q < nt) {
          float v = wave_sum(acc[x][q]);
          if (lane == 0 && e0 + x < E) ws.logits[static_cast<size_t>(t0 + q) * E + e0 + x] = v;
        }
      }
  }

  // ---- hand-off: the last workgroup to arrive runs phase 2
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(ws.counter, 1u, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == total_blocks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- phase 2a: top-k per token, one wave per token
  const int R = T * k;
  const int MW = (T + 63) / 64;
  int* s_ids = reinterpret_cast<int*>(smem);                                  // [T*k]
  unsigned long long* s_mask = reinterpret_cast<unsigned long long*>(
      smem + ((static_cast<size_t>(R) * 4 + 7) & ~static_cast<size_t>(7)));  // [E*MW]
  int* s_off = reinterpret_cast<int*>(s_mask + static_cast<size_t>(E) * MW);  // [E]

  for (int t = wave; t < T; t += 4) {
    int id = 0;
    float w = 0.f;
    select_token(ws.logits + static_cast<size_t>(t) * E, bias, E, k, rsf, &id, &w);
    if (lane < k) {
      const int r = t * k + lane;
      s_ids[r] = id;
      ws.ids[r] = id;
      ws.weights[r] = w;
      if (ids_out) ids_out[r] = id;
      if (w_out) w_out[r] = w;
    }
  }
  for (int i = threadIdx.x; i < E * MW; i += kThreads) s_mask[i] = 0ull;
  __syncthreads();

  // ---- phase 2b: route tables
  for (int r = threadIdx.x; r < R; r += kThreads) {
    const int e = s_ids[r], t = r / k;
    atomicOr(&s_mask[static_cast<size_t>(e) * MW + (t >> 6)], 1ull << (t & 63));
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
        for (int w = 0; w < MW; ++w) cnt += __popcll(s_mask[static_cast<size_t>(e) * MW + w]);
      packed[m] = (cnt << 11) | (cnt > 0 ? 1 : 0);
      local += packed[m];
    }
    int total = 0;
    int run = block_exclusive_scan(local, s_tmp, &total);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = 4 * threadIdx.x + m;
      if (e < E) {
        const int cnt = packed[m] >> 11;
        const int off = run >> 11, tidx = run & 0x7ff;
        s_off[e] = off;
        ws.counts[e] = cnt;
        ws.offsets[e] = off;
        if (cnt > 0) ws.touched[tidx] = e;
      }
      run += packed[m];
    }
    if (threadIdx.x == 0) {
      ws.offsets[E] = total >> 11;
      *ws.n_touched = total & 0x7ff;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += kThreads) {
    const int e = s_ids[r], t = r / k;
    const unsigned long long* m = s_mask + static_cast<size_t>(e) * MW;
    int rank = 0;
    for (int w = 0; w < (t >> 6); ++w) rank += __popcll(m[w]);
    rank += __popcll(m[t >> 6] & ((1ull << (t & 63)) - 1ull));
    const int pos = s_off[e] + rank;
    ws.perm[pos] = r;
    ws.inv[r] = pos;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(ws.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, hipStream_t s) {
  dim3 grid((d.E + 4 * kEpw - 1) / (4 * kEpw), (d.T + kTokB - 1) / kTokB);
  const int R = d.T * d.k, MW = (d.T + 63) / 64;
  size_t smem = ((static_cast<size_t>(R) * 4 + 7) & ~static_cast<size_t>(7)) +
                static_cast<size_t>(d.E) * MW * 8 + static_cast<size_t>(d.E) * 4;
  hipLaunchKernelGGL(router_kernel, grid, dim3(kThreads), smem, s,
                     static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(router_w),
                     bias, d.T, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out,
                     static_cast<uint32_t>(grid.x * grid.y));
  return hipGetLastError();
}

}  // namespace moe
