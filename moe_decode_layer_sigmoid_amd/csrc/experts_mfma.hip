// fp8 expert projections on the gfx950 matrix cores (the many-token regime).
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega builds the routed experts from
// w13 / w2 fp8 weights with 128x128 block scales (w13_weight_scale_inv,
// w2_weight_scale_inv; power-of-two e8m0 scales when that flag is set) and
// swiglu_limit, and picks a grouped kernel for larger token counts; the
// shared expert (SharedExpert) takes the same weight pair and limit.
//
// Each touched expert's weights are streamed from HBM once for all of its
// tokens.  A wave owns 16 NS weight rows (gate_up: 8 NS gate rows and the
// matching up rows; down: 16 NS consecutive output rows), so that each
// activation fragment it loads feeds NS MFMA subtiles, and walks the
// contraction dimension in 128-wide scale blocks.  The weights go from HBM
// straight to the wave's own LDS area (global_load_lds_dwordx4): eight
// consecutive lanes read the eight 16-byte pieces of one 128-byte block of
// a row, so every load instruction fetches whole 128-byte lines (the
// MFMA fragment order, four lanes per row, would fetch half lines and
// reach noticeably less of the HBM bandwidth).  The pieces land XOR-
// swizzled by row, so that the fragment reads from LDS spread over the
// banks.  Each lane then reads 32 fp8 bytes of its fragment row, converts
// them exactly to bf16, and v_mfma_f32_16x16x32_bf16 multiplies them with
// the bf16 activations of up to 16 tokens (one MFMA row per token; rows past
// the expert's token count repeat its last token and are never stored).
// Products are exact and the four MFMAs of a block sum in fp32; the block's
// partial is then scaled by the weight block scale and added to the fp32
// result, as the dequantise-then-multiply definition has it.
//
// The gate_up output (clamped SwiGLU) is stored as two bf16 planes,
// hi = bf16(a) and lo = bf16(a - hi), so that the down projection's
// activations keep 16 significant bits: down runs one MFMA on each plane.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, group g = l / 16,
// c = l % 16): A[c][8g + i] and B[8g + i][c] for i < 8; D[4g + i][c] for
// i < 4.  A lane's 32 bytes of a 128-wide block feed the four MFMAs of the
// block 8 bytes at a time (MFMA m takes contraction indices 32g + 8m + i),
// and its activation loads follow the same order, so A and B agree.
#include <algorithm>

#include "boundary_device.h"
#include "device_common.h"
#include "launch.h"
#include "sync_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kSubtileBlock = 2048;  // LDS bytes of one 128-wide block of 16 weight rows
constexpr unsigned kCpolNT = 2;    // non-temporal: weights are read once per step

// Issues the loads of one 128-wide block (byte offset kofs of every row) of
// the wave's 8 NI rows into `stage` (NI * 1024 bytes): load instruction i
// covers rows 8i .. 8i+7, whose start pointers lane l finds in row[i] (its
// row 8i + l / 8).  Lane l fetches piece (l % 8) ^ (l / 8) of its row and
// lands at stage + 1024 i + 16 l, so row r's piece p sits at slot
// p ^ (r % 8) of its 128 bytes.
template <int NI>
__device__ __forceinline__ void stage_block(const uint8_t* const row[NI], int kofs,
                                            unsigned char* stage) {
  const int lane = threadIdx.x & 63;
  const int piece = (lane & 7) ^ (lane >> 3);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_global_load_lds(row[i] + kofs + 16 * piece,
                                     (lds_void_t*)(stage + 1024 * i), 16, 0,
                                     kCpolNT);
}

// Piece p (16 bytes) of fragment row c of subtile s (rows 16 s + c) of a
// staged block.
__device__ __forceinline__ uint4 staged_piece(const unsigned char* stage, int s, int c, int p) {
  const int r8 = c & 7;
  return *reinterpret_cast<const uint4*>(stage + 1024 * (2 * s + (c >> 3)) + 128 * r8 +
                                         16 * (p ^ r8));
}

// Eight e4m3fn codes (two dwords, byte 0 first) -> eight bf16 (exact).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// dwords 2m, 2m+1 of a lane's 32 raw bytes (lo: bytes 0-15, hi: 16-31)
__device__ __forceinline__ bf16x8_t weight_frag(const uint4& lo, const uint4& hi, int m) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return fp8x8_to_bf16x8(w[2 * m], w[2 * m + 1]);
}

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return static_cast<uint16_t>(f32_to_bf16(f)); }

// Each wave walks the contraction in blocks of 128 columns.  If every wave
// started at block 0, the waves would read the same block columns at once:
// up to this many tokens the launches' workgroups all start in about one
// round and then drain unevenly; and where the gate_up rows are a power of
// two bytes long (H = 4096) those columns of all rows share the same few
// memory channels, at any token count (the down tiles follow the same rule).
// There each wave starts at its own
// block (its id modulo the block count) and wraps around; the order of a
// wave's blocks is fixed by the grid, so results stay deterministic.
// Measured at H = 4096, E = 128: 64 tokens 472 -> 430 us, 128 tokens 515 ->
// 472 us, 256 tokens 649 -> 633 us.  Otherwise, with more tokens, later
// workgroups start staggered anyway, and the rotation only scatters the
// accesses of neighbouring waves (measured slower at H = 6144 with 64 and
// 128 tokens; rotating by the down rows' length, I = 2048 there, changed
// nothing).
constexpr int kRotateMaxTokens = 32;

__device__ __forceinline__ int first_block(int T, int H, int wave, int KB, int bx, int by) {
  if (T > kRotateMaxTokens && (H & (H - 1)) != 0) return 0;
  return (bx * kWaves + wave + 5 * by) % KB;
}

// Block i of a wave's walk (i past the end: the last block, whose scale the
// caller zeroes).
__device__ __forceinline__ int block_at(int i, int KB, int rot) {
  const int b = min(i, KB - 1) + rot;
  return b >= KB ? b - KB : b;
}

// A shared activation tile (launches of one row kind): the 16 token rows
// of one 128-column block, 256 bytes each, loaded once per workgroup
// instead of once per wave.  Lane l of wave w loads tile row
// r = 4 w + l / 16 and lands at piece l % 16 of it; it fetches piece
// (l % 16) ^ r of the row, so piece p of row r sits at slot p ^ r and the
// fragment reads (16 rows, one piece each) spread over the banks.
constexpr int kActTile = 16 * 256;

__device__ __forceinline__ uint4 act_piece(const unsigned char* tile, int r, int p) {
  return *reinterpret_cast<const uint4*>(tile + 256 * r + 16 * (p ^ r));
}

// What one grid row works on (uniform).  Rows [0, SP) are the shared
// expert, one 16 * GR-token pass each (they run in parallel); the rows after
// them are the touched-expert slots, each taking all of its expert's tokens
// in passes of 16 * GR.  Tokens [p_begin, p_end) of the row's expert; base =
// the expert's first permuted position (0 for the shared expert, whose
// positions are the tokens themselves).
struct Slot {
  bool shared;
  int e, base, p_begin, p_end;
};

template <int GR>
__device__ __forceinline__ bool slot_of(int T, int SP, const Workspace& ws, int y, Slot* s) {
  if (y < SP) {
    const int p = y * 16 * GR;
    *s = {true, 0, 0, p, min(T, p + 16 * GR)};
    return p < T;
  }
  // the router's slot record: expert (-1: none this step), count, base
  const int4 rec =
      *reinterpret_cast<const int4*>(ws.slot_tab + static_cast<size_t>(y - SP) * kSlotInts);
  if (rec.x < 0) return false;
  *s = {false, rec.x, rec.z, 0, rec.y};
  return true;
}

// gate_up + clamped SwiGLU.  Wave: SwiGLU outputs [i0, i0 + 8 NS) of one
// expert for all its tokens (NS 16-row subtiles of weights: NS / 2 of gate
// rows, then the NS / 2 matching subtiles of up rows); writes the hi / lo
// bf16 planes of act[(base + q) * I + i].  U = scale blocks per round of
// loads; GR = 16-token groups per pass over the weights.
// ROWS: kAllRows (shared passes and touched experts, chosen per row at run
// time) or only one kind, fixed at compile time.
// The tile of workgroup (bx, by) of that grid; returns whether it worked
// (false: an empty slot or a tile past the row's end).  C: the SwiGLU planes
// are written with agent-scope atomic stores (write-through, two bf16 of
// neighbouring lanes per 32-bit store), for readers in the same launch: a
// plain store leaves the line in the writer's L2, possibly filled with stale
// bytes of the part other workgroups write.
template <int NS, int U, int GR, bool E8, int ROWS, bool C = false, bool SA = false>
__device__ __forceinline__ bool gate_up_tile(
    int bx, int by, unsigned char* smem, const uint16_t* __restrict__ hidden,
    const uint8_t* __restrict__ w13, const void* __restrict__ scale13,
    const uint8_t* __restrict__ sw13, const void* __restrict__ sscale13, int H, int I_r, int Is,
    int k, int T, int SP, const Workspace& ws, float limit) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  constexpr int NH = NS / 2;  // gate (and up) subtiles
  // SA: activation tiles shared through LDS (launches of one row kind)
  static_assert(!SA || (U == 1 && ROWS != kAllRows), "a shared tile holds one block");
  const int i0 = (bx * kWaves + wave) * 16 * NH;
  Slot sl;
  if (!slot_of<GR>(T, SP, ws, by, &sl)) return false;
  const bool shared = ROWS == kAllRows ? sl.shared : ROWS == kSharedRows;
  const int I = shared ? Is : I_r;
  // a workgroup covers 32 NS outputs, a divisor of 128: uniform over it
  if (i0 >= I) return false;
  const void* scale = shared ? sscale13 : scale13;
  constexpr int SB = NS * kSubtileBlock;  // stage bytes of one block
  unsigned char* stage = smem + wave * U * SB;
  // SA: two rounds of GR tiles of kActTile bytes (double-buffered)
  unsigned char* atile = smem + kWaves * U * SB;
  int rd = 0;  // rounds so far, over all passes: the tiles' buffer
  const int KB = H / kBlock;
  // with shared tiles every wave of the workgroup walks the same blocks
  const int rot = first_block(T, H, SA ? 0 : wave, KB, bx, by);
  const uint8_t* W = shared ? sw13 : w13 + static_cast<size_t>(sl.e) * 2 * I * H;
  // load rows: instructions [0, NS) = gate rows i0 .. i0 + 8 NS - 1, then up
  const uint8_t* lrow[2 * NS];
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i)
    lrow[i] = W + static_cast<size_t>((i < NS ? i0 : I + i0 - 8 * NS) + 8 * i + (lane >> 3)) * H;
  const size_t sb = static_cast<size_t>(sl.e) * (2 * I / kBlock) * KB;
  const size_t sg0 = sb + static_cast<size_t>(i0 / kBlock) * KB;
  const size_t su0 = sb + static_cast<size_t>((I + i0) / kBlock) * KB;
  uint16_t* act_hi = reinterpret_cast<uint16_t*>(shared ? ws.act_s : ws.act);
  const size_t plane = static_cast<size_t>(shared ? T : T * k) * I;
  uint16_t* act_lo = act_hi + plane;

  for (int p0 = sl.p_begin; p0 < sl.p_end; p0 += 16 * GR) {
    const int G = min(GR, (sl.p_end - p0 + 15) / 16);
    // xrow: the lane's own fragment row; SA: the tile row this lane loads
    // (tile row 4 wave + lane / 16, 16-byte piece (lane % 16) ^ row)
    const uint16_t* xrow[GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      const int r = SA ? 4 * wave + (lane >> 4) : c;
      const int q = min(p0 + gr * 16 + r, sl.p_end - 1);
      const int t = shared ? q : ws.perm[sl.base + q] / k;
      xrow[gr] = hidden + static_cast<size_t>(t) * H + (SA ? 8 * ((lane & 15) ^ r) : 32 * g);
    }
    f32x4_t fg[GR][NH], fu[GR][NH];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        fg[gr][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        fu[gr][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int kb0 = 0; kb0 < KB; kb0 += U) {
      float sg[U], su[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int kb = block_at(kb0 + j, KB, rot);  // a block past the end gets scale 0
        stage_block<2 * NS>(lrow, kb * kBlock, stage + j * SB);
        const float a = load_scale<E8>(scale, sg0 + kb);
        const float b = load_scale<E8>(scale, su0 + kb);
        sg[j] = kb0 + j < KB ? a : 0.f;
        su[j] = kb0 + j < KB ? b : 0.f;
      }
      unsigned char* at = atile + (rd & 1) * GR * kActTile;
      if (SA) {
        // the block's activation tiles, one load per lane and group, into
        // the buffer every wave last read two rounds ago (before its barrier
        // of the previous round)
        const int kb = block_at(kb0, KB, rot);
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
          __builtin_amdgcn_global_load_lds(xrow[gr] + kb * kBlock,
                                           (lds_void_t*)(at + gr * kActTile + 1024 * wave), 16, 0,
                                           0);
        }
      }
      // every load of the round is issued before the first wait
      asm volatile("" ::: "memory");
      uint4 xa[GR][U][4];
      if (!SA) {
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
#pragma unroll
          for (int j = 0; j < U; ++j) {
            const int kb = block_at(kb0 + j, KB, rot);
#pragma unroll
            for (int m = 0; m < 4; ++m)
              xa[gr][j][m] = *reinterpret_cast<const uint4*>(xrow[gr] + kb * kBlock + 8 * m);
          }
        }
      }
      // The staged weights land in LDS through the loads' own path: the
      // compiler does not order the LDS reads below after them, so wait
      // for every load of the wave here (the activation loads above are
      // issued by then).
      wait_memory();
      if (SA) {
        __syncthreads();  // every wave's part of the tiles is in LDS
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
#pragma unroll
          for (int m = 0; m < 4; ++m) xa[gr][0][m] = act_piece(at + gr * kActTile, c, 4 * g + m);
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const unsigned char* st = stage + j * SB;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const uint4 g0 = staged_piece(st, h, c, 2 * g), g1 = staged_piece(st, h, c, 2 * g + 1);
          const uint4 u0 = staged_piece(st, NH + h, c, 2 * g),
                      u1 = staged_piece(st, NH + h, c, 2 * g + 1);
          f32x4_t pg[GR], pu[GR];
#pragma unroll
          for (int gr = 0; gr < GR; ++gr) {
            pg[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            pu[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            // each weight fragment is converted once for every group of the pass
            const bf16x8_t wg = weight_frag(g0, g1, m), wu = weight_frag(u0, u1, m);
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) {
              if (gr >= G) break;
              const bf16x8_t a = as_bf16x8(xa[gr][j][m]);
              pg[gr] = mfma(a, wg, pg[gr]);
              pu[gr] = mfma(a, wu, pu[gr]);
            }
          }
#pragma unroll
          for (int gr = 0; gr < GR; ++gr) {
            if (gr >= G) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              fg[gr][h][i] = fmaf(sg[j], pg[gr][i], fg[gr][h][i]);
              fu[gr][h][i] = fmaf(su[j], pu[gr][i], fu[gr][h][i]);
            }
          }
        }
      }
      // the next round's loads overwrite the stage: its reads must be done
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      ++rd;
    }
    // lane holds tokens p0 + 16 gr + 4 g + i of SwiGLU outputs i0 + 16 h + c
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      if (gr >= G) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = p0 + gr * 16 + 4 * g + i;
        if (q < sl.p_end) {
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const float a = clamped_swiglu(fg[gr][h][i], fu[gr][h][i], limit);
            const uint16_t hi = bf16_bits(a);
            const uint16_t lo = bf16_bits(a - bf16_to_f32(hi));
            const size_t o = static_cast<size_t>(sl.base + q) * I + i0 + 16 * h + c;
            if (C) {
              // lanes c and c ^ 1 hold neighbouring outputs of the same token
              // (the condition above is uniform over the 16 lanes of g)
              const uint32_t hi2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), 1));
              const uint32_t lo2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), 1));
              if ((c & 1) == 0) {
                st_u32<true>(reinterpret_cast<uint32_t*>(act_hi + o), hi | (hi2 << 16));
                st_u32<true>(reinterpret_cast<uint32_t*>(act_lo + o), lo | (lo2 << 16));
              }
            } else {
              act_hi[o] = hi;
              act_lo[o] = lo;
            }
          }
        }
      }
    }
  }
  return true;
}

template <int NS, int U, int GR, bool E8, int ROWS, bool SA>
__global__ __launch_bounds__(kThreads) void gate_up_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ w13,
    const void* __restrict__ scale13, const uint8_t* __restrict__ sw13,
    const void* __restrict__ sscale13, int H, int I_r, int Is, int k, int T, int SP,
    Workspace ws, float limit) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  gate_up_tile<NS, U, GR, E8, ROWS, false, SA>(blockIdx.x, blockIdx.y, smem, hidden, w13,
                                               scale13, sw13, sscale13, H, I_r, Is, k, T, SP, ws,
                                               limit);
}

// down projection.  Wave: output rows [h0, h0 + 16 NS) of one expert for all
// its tokens, from the hi / lo activation planes; row q goes to
// out[perm[base + q] * H] (routed: the route index t*k + j) or out[q * H]
// (shared).
// The tile of workgroup (bx, by) of that grid.  wait() runs once, after the
// first round of weight loads is issued and before the first activation is
// read (every wave of the workgroup calls it); the kernel of its own passes
// NoWait.
// Activation tile buffers of a shared-tile (SA) down launch: two (one
// barrier per block) where the workgroup's LDS stays within half a CU's
// 160 KB, so that two workgroups fit; else one, refilled after a second
// barrier.  Measured on MI355X at H = 4096, E = 128, 256 tokens (two groups,
// 128 rows per wave): double-buffered tiles took 96 KB and one workgroup per
// CU, 574 -> 611 us per layer.
__host__ __device__ constexpr int dn_sa_buffers(int NS, int U, int GR) {
  return kWaves * U * NS * kSubtileBlock + 4 * GR * kActTile <= 80 * 1024 ? 2 : 1;
}

template <int NS, int U, int GR, bool E8, int ROWS, typename Wait, bool SA = false,
          bool CST = false>
__device__ __forceinline__ void down_tile(
    int bx, int by, unsigned char* smem, const uint8_t* __restrict__ w2,
    const void* __restrict__ scale2, const uint8_t* __restrict__ sw2,
    const void* __restrict__ sscale2, int H, int I_r, int Is, int k, int T, int SP,
    const Workspace& ws, Wait wait) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  // SA: activation tiles shared through LDS (launches of one row kind)
  static_assert(!SA || (U == 1 && ROWS != kAllRows), "a shared tile holds one block");
  const int h0 = (bx * kWaves + wave) * 16 * NS;
  Slot sl;
  if (!slot_of<GR>(T, SP, ws, by, &sl)) return;
  // past the last row: with shared tiles the wave still loads its part of
  // them and meets the workgroup's barriers, but streams no weights
  const bool live = h0 < H;
  if (!SA && !live) return;
  const bool shared = ROWS == kAllRows ? sl.shared : ROWS == kSharedRows;
  const int I = shared ? Is : I_r;
  const void* scale = shared ? sscale2 : scale2;
  constexpr int SB = NS * kSubtileBlock;
  unsigned char* stage = smem + wave * U * SB;
  // SA: GR x (hi, lo) tiles, double-buffered where two workgroups per CU
  // still fit (dn_sa_buffers)
  constexpr int NBUF = dn_sa_buffers(NS, U, GR);
  unsigned char* atile = smem + kWaves * U * SB;
  int rd = 0;  // rounds so far, over all passes: the tiles' buffer
  const int KB = I / kBlock;
  const int rot = first_block(T, H, SA ? 0 : wave, KB, bx, by);
  const uint8_t* W = shared ? sw2 : w2 + static_cast<size_t>(sl.e) * H * I;
  const uint8_t* lrow[2 * NS];
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i)
    lrow[i] = W + static_cast<size_t>(h0 + 8 * i + (lane >> 3)) * I;
  const size_t s0 = static_cast<size_t>(sl.e) * (H / kBlock) * KB +
                    static_cast<size_t>(h0 / kBlock) * KB;
  const uint16_t* act_hi = reinterpret_cast<const uint16_t*>(shared ? ws.act_s : ws.act);
  const size_t plane = static_cast<size_t>(shared ? T : T * k) * I;
  const uint16_t* act_lo = act_hi + plane;
  float* out = shared ? ws.y_s : ws.rows;
  bool waited = false;

  for (int p0 = sl.p_begin; p0 < sl.p_end; p0 += 16 * GR) {
    const int G = min(GR, (sl.p_end - p0 + 15) / 16);
    // arow: the lane's own fragment row; SA: the tile row this lane loads
    size_t arow[GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      const int r = SA ? 4 * wave + (lane >> 4) : c;
      const int q = min(p0 + gr * 16 + r, sl.p_end - 1);
      arow[gr] = static_cast<size_t>(sl.base + q) * I + (SA ? 8 * ((lane & 15) ^ r) : 32 * g);
    }
    f32x4_t f[GR][NS];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr)
#pragma unroll
      for (int s = 0; s < NS; ++s) f[gr][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < KB; kb0 += U) {
      float sc[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int kb = block_at(kb0 + j, KB, rot);
        if (live) stage_block<2 * NS>(lrow, kb * kBlock, stage + j * SB);
        const float s = live ? load_scale<E8>(scale, s0 + kb) : 0.f;
        sc[j] = kb0 + j < KB ? s : 0.f;
      }
      asm volatile("" ::: "memory");
      if (!waited) {  // uniform
        wait();
        waited = true;
      }
      unsigned char* at = atile + (NBUF == 2 ? (rd & 1) * 2 * GR * kActTile : 0);
      if (SA) {
        // the block's hi and lo activation tiles: into the buffer every wave
        // last read two rounds ago (as in gate_up_tile), or into the one
        // buffer once every wave is done reading the previous block's
        if (NBUF == 1) __syncthreads();
        const int kb = block_at(kb0, KB, rot);
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
          unsigned char* t = at + 2 * gr * kActTile + 1024 * wave;
          __builtin_amdgcn_global_load_lds(act_hi + arow[gr] + kb * kBlock, (lds_void_t*)t, 16, 0,
                                           0);
          __builtin_amdgcn_global_load_lds(act_lo + arow[gr] + kb * kBlock,
                                           (lds_void_t*)(t + kActTile), 16, 0, 0);
        }
      }
      uint4 ah[GR][U][4], al[GR][U][4];
      if (!SA) {
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
#pragma unroll
          for (int j = 0; j < U; ++j) {
            const int kb = block_at(kb0 + j, KB, rot);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              ah[gr][j][m] =
                  *reinterpret_cast<const uint4*>(act_hi + arow[gr] + kb * kBlock + 8 * m);
              al[gr][j][m] =
                  *reinterpret_cast<const uint4*>(act_lo + arow[gr] + kb * kBlock + 8 * m);
            }
          }
        }
      }
      wait_memory();  // the staged weights are in LDS (see gate_up_tile)
      if (SA) {
        __syncthreads();  // every wave's part of the tiles is in LDS
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            ah[gr][0][m] = act_piece(at + 2 * gr * kActTile, c, 4 * g + m);
            al[gr][0][m] = act_piece(at + (2 * gr + 1) * kActTile, c, 4 * g + m);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (!live) break;
        const unsigned char* st = stage + j * SB;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint4 a0 = staged_piece(st, s, c, 2 * g), a1 = staged_piece(st, s, c, 2 * g + 1);
          f32x4_t p[GR];
#pragma unroll
          for (int gr = 0; gr < GR; ++gr) p[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            // each weight fragment is converted once for every group of the pass
            const bf16x8_t wa = weight_frag(a0, a1, m);
#pragma unroll
            for (int gr = 0; gr < GR; ++gr) {
              if (gr >= G) break;
              p[gr] = mfma(as_bf16x8(ah[gr][j][m]), wa, p[gr]);
              p[gr] = mfma(as_bf16x8(al[gr][j][m]), wa, p[gr]);
            }
          }
#pragma unroll
          for (int gr = 0; gr < GR; ++gr) {
            if (gr >= G) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) f[gr][s][i] = fmaf(sc[j], p[gr][i], f[gr][s][i]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): stage reads done
      ++rd;
    }
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      if (gr >= G) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = p0 + gr * 16 + 4 * g + i;
        if (live && q < sl.p_end) {
          const int o = shared ? q : ws.perm[sl.base + q];
          float* row = out + static_cast<size_t>(o) * H + h0 + c;
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            // CST: read in this launch (the merged launch's boundary)
            if (CST)
              st_f32<true>(row + 16 * s, f[gr][s][i]);
            else
              row[16 * s] = f[gr][s][i];
          }
        }
      }
    }
  }
}

struct NoWaitMfma {
  __device__ void operator()() const {}
};

template <int NS, int U, int GR, bool E8, int ROWS, bool SA>
__global__ __launch_bounds__(kThreads) void down_mfma_kernel(
    const uint8_t* __restrict__ w2, const void* __restrict__ scale2,
    const uint8_t* __restrict__ sw2, const void* __restrict__ sscale2, int H, int I_r, int Is,
    int k, int T, int SP, Workspace ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  down_tile<NS, U, GR, E8, ROWS, NoWaitMfma, SA>(blockIdx.x, blockIdx.y, smem, w2, scale2, sw2,
                                                 sscale2, H, I_r, Is, k, T, SP, ws,
                                                 NoWaitMfma());
}

// Per wave: NS 16-row weight subtiles, U scale blocks per round of loads,
// one 16-token group per pass (the shared expert gets one grid row per 16
// tokens, so that its passes run in parallel).
// The routed-only down launch (above kMergeSharedMaxTokens, several tokens
// per expert) takes 128 rows per wave: each activation fragment then feeds
// eight weight subtiles (measured 8% faster there; no gain at 64 tokens).
// Every pass streams the expert's weights again, so once the routes average
// kGr2MinMean tokens per expert (many experts then hold more than 16) the
// routed-only launches take two 16-token groups per pass: the extra
// accumulators cost occupancy, which is a net loss below that mean (measured
// at H = 4096, E = 128: 256 tokens 827 -> 647 us, 192 tokens 643 -> 578 us,
// 128 tokens 514 -> 517 us; neutral at H = 6144, E = 256 up to 256 tokens).
// Both tiles convert each staged weight fragment once for both groups
// (256 tokens 632 -> 609 us for gate_up, though its fp32-scale kernel then
// holds 144 VGPRs; then 611 -> 591 us for down).  With that, two groups pay
// from a mean of 10 (160 tokens at E = 128: 523 -> 510 us) and still lose
// at 8 (128 tokens: 472 -> 483 us) and 6 (96 tokens: 450 -> 457 us).
constexpr int kNsGu = 4, kUGu = 1;
// The routed-only launches with two groups per pass and shared activation
// tiles give each wave 64 gate + 64 up rows instead: a workgroup covers 256
// outputs, so fewer workgroups re-read each expert's token rows.  Measured
// on MI355X at H = 4096, E = 128 (us per layer): 256 tokens 534.5 -> 520.0,
// 192 tokens 504.1 -> 503.2; with one group per pass it lost (128 tokens
// +1%, H = 6144 at 128 and 256 tokens +2.5% and +1.7%).
constexpr int kNsGuWide = 8;
constexpr int kNsDn = 4, kNsDnRouted = 8, kUDn = 1;
constexpr int kGR = 1;  // 16-token groups per pass
constexpr int kGr2MinMean = 10;
bool routed_gr2(const LayerDims& d) { return d.T * d.k >= kGr2MinMean * d.E; }
// The routed-only launches load each 16-token activation tile once per
// workgroup into LDS (SA), not once per wave: from a mean of
// kSharedActMinMean tokens per expert with two groups per pass, and of
// kSharedActMinMean1 with one.  Counters of the routed gate_up launch showed
// every CU issuing about 0.1 L2 read request per clock whatever the kernel,
// activation hits included: at H = 4096, E = 128 the hits were 18% of the
// requests at 128 tokens and 33% at 256 (9% at H = 6144, E = 256, 128
// tokens), a share the weight misses lose.  The tiles alternate between two
// buffers, so a block needs one workgroup barrier (the down launch keeps one
// buffer, and a second barrier, where two would leave room for only one
// workgroup per CU: dn_sa_buffers).  Measured on MI355X (us per layer,
// against the per-wave loads): H = 4096, E = 128: 96 tokens 454.4 -> 452.9,
// 128 tokens 474.5 -> 463.4, 160 tokens 514.1 -> 505.6, 192 tokens
// 536.0 -> 525.7, 256 tokens 574.5 -> 562.0; H = 6144, E = 256: 128 tokens
// 1548.7 -> 1540.1, 256 tokens 1703.5 -> 1665.9.  With two barriers per
// block the tiles had paid only from 16 tokens per expert.
constexpr int kSharedActMinMean = 10;
static_assert(kSharedActMinMean >= kGr2MinMean, "this threshold is for two groups per pass");
bool routed_sa(const LayerDims& d) { return d.T * d.k >= kSharedActMinMean * d.E; }
constexpr int kSharedActMinMean1 = 4;
// The shared expert's own launches (beside the routed-only ones, above
// kMergeSharedMaxTokens tokens) take two 16-token groups per pass, with
// shared activation tiles, from kSharedGr2MinTokens tokens on: each pass
// streams the shared weights again, 16 passes at 256 tokens with one group.
// Measured on MI355X (us per layer): H = 4096, E = 128: 160 tokens
// 505.0 -> 495.2, 192 tokens 523.9 -> 502.3, 256 tokens 560.1 -> 532.2;
// H = 6144, E = 256, 192 tokens 1622.6 -> 1613.0.  From 65 tokens on, the
// shared passes' fewer and longer workgroups delayed the join: 96 tokens
// 453.8 -> 456.8, 128 tokens 462.1 -> 464.7, and 1539 -> 1553 at H = 6144.
constexpr int kSharedGr2MinTokens = 160;
int shared_gr(const LayerDims& d) { return d.T >= kSharedGr2MinTokens ? 2 : kGR; }
bool routed_sa1(const LayerDims& d) { return d.T * d.k >= kSharedActMinMean1 * d.E; }
constexpr size_t kLdsGu = static_cast<size_t>(kWaves) * kUGu * kNsGu * kSubtileBlock;

template <bool E8, int ROWS, int GR = kGR, int NS = kNsGu, bool SA = false>
void launch_gu(dim3 grid, hipStream_t s, const uint16_t* x, const uint8_t* w, const void* scale,
               const uint8_t* sw, const void* sscale, const LayerDims& d, int SP,
               const Workspace& ws, hipEvent_t evb, hipEvent_t eve) {
  const size_t lds = static_cast<size_t>(kWaves) * kUGu * NS * kSubtileBlock +
                     (SA ? static_cast<size_t>(2 * GR) * kActTile : 0);
  MOE_LAUNCH((gate_up_mfma_kernel<NS, kUGu, GR, E8, ROWS, SA>), grid, dim3(kThreads), lds, s,
             evb, eve, x, w, scale, sw, sscale, d.H, d.I, d.Is, d.k, d.T, SP, ws, d.limit);
}

template <int NS, bool E8, int ROWS, int GR = kGR, bool SA = false>
void launch_dn(int R, hipStream_t s, const uint8_t* w, const void* scale, const uint8_t* sw,
               const void* sscale, const LayerDims& d, int SP, const Workspace& ws) {
  const int per_wg = kWaves * 16 * NS;  // output rows per workgroup
  const dim3 grid((d.H + per_wg - 1) / per_wg, SP + R);
  const size_t lds = static_cast<size_t>(kWaves) * kUDn * NS * kSubtileBlock +
                     (SA ? static_cast<size_t>(2 * dn_sa_buffers(NS, kUDn, GR) * GR) * kActTile
                         : 0);
  hipLaunchKernelGGL((down_mfma_kernel<NS, kUDn, GR, E8, ROWS, SA>), grid, dim3(kThreads), lds,
                     s, w, scale, sw, sscale, d.H, d.I, d.Is, d.k, d.T, SP, ws);
}

// The gate_up and down tiles of the merged launch (shared passes and touched
// slots, up to kMergeSharedMaxTokens tokens) and the boundary as one launch:
// workgroups [0, n_gu) are the gate_up tiles (row-major over grid rows), then
// the n_dn down tiles, then T * bnd_ns boundary slices (boundary_device.h),
// which wait until every down tile has written its rows (write-through
// stores) and counted itself.  A down tile issues its first round of weight
// loads, then waits
// until every gate_up tile of its row has published its SwiGLU planes, so
// the down weights stream while the gate_up tiles drain (their waves end over
// a wide window: 130 to 187 us at 16 tokens).  A gate_up tile writes its
// SwiGLU planes with write-through (agent-scope atomic) stores, waits for
// them, and then bumps its row's count; the down tile reads the planes with
// plain loads (no L2 holds their lines when the launch starts, and nothing
// reads them before the count is complete).  A workgroup waits only for workgroups of
// lower index, which the dispatcher starts first; waits are bounded (the
// sticky error word).  The router launch zeroes the counts.
constexpr uint32_t kGChainSpin = 1u << 17;

// Counter line of grid row y: the shared passes on the flag lines, the
// touched slots on their gate_up count lines.
__device__ __forceinline__ int gchain_line(int y, int SP) {
  return y < SP ? kSyncFlags + y : sync_gu_cnt(y - SP);
}

template <bool E8>
__global__ __launch_bounds__(kThreads, 4) void grouped_chain_kernel(GChainArgs a, Workspace ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const Sync sy{ws.sync};
  const int it = blockIdx.x;
  if (it < a.n_gu) {
    const int by = it / a.gx, bx = it - by * a.gx;
    if (gate_up_tile<kNsGu, kUGu, kGR, E8, kAllRows, true>(
            bx, by, smem, a.hidden, a.w13, a.w13_scale, a.sw13, a.sw13_scale, a.H, a.I, a.Is,
            a.k, a.T, a.SP, ws, a.limit))
      bump(sy, gchain_line(by, a.SP));
    return;
  }
  const int v = it - a.n_gu;
  if (v < a.n_dn) {
    const int by = v / a.dx, bx = v - by * a.dx;
    // the row's gate_up tiles (a tile covers kWaves * 8 * kNsGu SwiGLU outputs)
    const uint32_t target = static_cast<uint32_t>((by < a.SP ? a.Is : a.I) / (kWaves * 8 * kNsGu));
    auto wait = [&]() { wait_count(sy, gchain_line(by, a.SP), 1, target, kGChainSpin); };
    if (a.bnd_ns > 0) {
      // the boundary is in this launch: rows written through, and counted
      down_tile<kNsDn, kUDn, kGR, E8, kAllRows, decltype(wait), false, true>(
          bx, by, smem, a.w2, a.w2_scale, a.sw2, a.sw2_scale, a.H, a.I, a.Is, a.k, a.T, a.SP,
          ws, wait);
      bump(sy, kSyncExit0 + v % kSyncExitLines);
    } else {
      down_tile<kNsDn, kUDn, kGR, E8, kAllRows, decltype(wait), false, false>(
          bx, by, smem, a.w2, a.w2_scale, a.sw2, a.sw2_scale, a.H, a.I, a.Is, a.k, a.T, a.SP,
          ws, wait);
    }
    return;
  }
  // ---- the boundary (the last T * bnd_ns workgroups), after every down tile
  const int b = v - a.n_dn;
  const BndArgs bn{a.residual, a.gamma, a.out, a.residual_out, a.moe_out, a.H, a.k, a.Is,
                   a.bnd_ns, a.eps, ws.epi_part, sy.line(kSyncError)};
  constexpr int kCpt = kBndCols / kBndThreads;
  boundary_slice<false, kCpt>(bn, ws, b / a.bnd_ns, b % a.bnd_ns, [&]() {
    wait_count(sy, kSyncExit0, kSyncExitLines, static_cast<uint32_t>(a.n_dn), kGChainSpin);
  }, StepTail{});
}

// Dense layers (no routed experts).  The MLP is one expert of I_s rows that
// every token takes, so a 16-token pass of the tiles above has only I_s / 64
// gate_up and H / 64 down workgroups (128 and 64 at I_s = 8192, H = 4096):
// too few loads in flight for HBM.  The kernels below split the contraction
// over workgroups instead.  Each workgroup owns a row tile (gate_up: 64
// SwiGLU outputs, wave w the 16 gate rows and the matching 16 up rows of
// outputs 16 w ..; down: 128 output rows, wave w rows 32 w ..) over one of S
// contiguous ranges of the contraction, and its four waves walk the same
// 128-column blocks: the weights go to each wave's own LDS area, the
// activations of a block are staged into LDS once per workgroup and read by
// all four waves.  A CU serves L1 misses (L2 hits included) at about one
// request per ten clocks, so activations read once per wave would cost as
// many requests as the weights from 16 tokens on; staged once per workgroup
// they cost a quarter of that.  The S workgroups of a tile write their fp32
// partial sums; the last of them to arrive adds the ranges in range order
// (results stay deterministic) and finishes the tile: the clamped SwiGLU into
// the hi / lo planes, or the down output rows.  Every 16 GR-token pass
// streams the weights again; workgroup b runs on XCD b % 8 (the dispatcher's
// round robin), so the grid puts all passes of a unit on one XCD and next to
// each other in dispatch order, where the later passes find the weight lines
// in that XCD's L2.  A layer of one token group (at most 16 tokens) runs its
// gate_up on dense_gate_up_waves_mfma_kernel instead, which hands nothing
// between workgroups.
constexpr int kDenseGuOuts = 64;     // SwiGLU outputs per gate_up workgroup (16 per wave)
constexpr int kDenseDnRows = 128;    // down output rows per workgroup (32 per wave)
constexpr int kDenseMaxGroups = 4;   // 16-token groups per workgroup
constexpr int kDenseGuMaxSplits = 4;
constexpr int kDenseDnMaxSplits = 8;
constexpr int kDenseMinGrid = 512;   // workgroups a launch aims for: two per CU
constexpr int kXcds = 8;
constexpr int kActBlock = 16 * kBlock * 2;  // LDS bytes of 16 tokens x 128 bf16 columns

// blocks [*b0, *b0 + *nb) of range u of n equal contiguous ranges over KB blocks
__device__ __forceinline__ void k_range(int u, int n, int KB, int* b0, int* nb) {
  const int a = u * KB / n, b = (u + 1) * KB / n;
  *b0 = a;
  *nb = b - a;
}

// Workgroup b -> (unit, pass), with every pass of a unit on one XCD and
// adjacent in dispatch order (the grid holds ceil(units / 8) * 8 * P).
__device__ __forceinline__ void xcd_tile_pass(int b, int P, int* unit, int* pass) {
  const int x = b % kXcds, r = b / kXcds;
  *pass = r % P;
  *unit = (r / P) * kXcds + x;
}

// Block i of a workgroup's range (i past the end: the last, whose scale the
// caller zeroes), rotated by rot so that the workgroups' first loads spread
// over the row's columns.
__device__ __forceinline__ int range_block(int i, int b0, int nb, int rot) {
  const int j = min(i, nb - 1) + rot;
  return b0 + (j >= nb ? j - nb : j);
}

// The weight side of MFMA m for lane (g, c): the 8 bytes at columns
// 32 m + 8 g of row c of the staged block, half (g & 1) of staged piece
// 2 m + (g >> 1) (pieces sit at slot p ^ (row % 8), see stage_block).
__device__ __forceinline__ uint2 staged_half(const unsigned char* stage, int s, int c, int m,
                                             int g) {
  const int r8 = c & 7, p = 2 * m + (g >> 1);
  return *reinterpret_cast<const uint2*>(stage + 1024 * (2 * s + (c >> 3)) + 128 * r8 +
                                         16 * (p ^ r8) + 8 * (g & 1));
}

// Activations of one 128-column block for one 16-token group, staged in LDS
// (kActBlock bytes): token row r at 256 r, its 16-byte piece p at slot
// p ^ r.  Wave w stages rows 4 w .. 4 w + 3 with one load instruction: lane
// l takes row r = 4 w + l / 16 and lands at slot l % 16, so it fetches piece
// (l % 16) ^ r; the 16 lanes of a row fetch its two whole 128-byte lines.
// act_src gives lane l's source (row start + 8 ((l % 16) ^ r) elements).
__device__ __forceinline__ const uint16_t* act_src(const uint16_t* row_start) {
  const int lane = threadIdx.x & 63;
  const int r = 4 * static_cast<int>(threadIdx.x >> 6) + (lane >> 4);
  return row_start + 8 * ((lane & 15) ^ r);
}
__device__ __forceinline__ int act_row() {
  return 4 * static_cast<int>(threadIdx.x >> 6) + ((threadIdx.x & 63) >> 4);
}
__device__ __forceinline__ void stage_act(const uint16_t* src, unsigned char* blk) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(blk + 1024 * (threadIdx.x >> 6)), 16, 0,
                                   0);
}
// The activation side of MFMA m for lane (g, c): token c, columns
// 32 m + 8 g .. + 7 (piece 4 m + g); the 16 lanes of one g read 16
// different slots, so the read spreads over the banks.
__device__ __forceinline__ bf16x8_t act_frag(const unsigned char* blk, int c, int m, int g) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(blk + 256 * c + 16 * ((4 * m + g) ^ c)));
}

// Contraction ranges of a dense launch: enough workgroups for two per CU,
// at most max_s, two blocks per range at least.
__host__ __device__ inline int dense_splits(int tiles, int P, int KB, int max_s) {
  int S = (kDenseMinGrid + tiles * P - 1) / (tiles * P);
  S = S < max_s ? S : max_s;
  S = S < KB / 2 ? S : KB / 2;
  return S > 1 ? S : 1;
}

// The S workgroups of (unit, pass) hand their sums to the last of them:
// each stores its NV float4 per thread (write-through; nv of them hold
// tokens) into its range's slot of `part`, then counts itself on `cnt`; the
// last one resets the count and returns true with v[] replaced by the sums
// over the ranges in range order (its own from registers).  The others
// return false.  The loads of the sums are issued before their adds, up to
// 16 per thread at a time: slots past S or nv are read too (they are in the
// buffer) and not used.
template <int NV, int MAXS>
__device__ __forceinline__ bool dense_hand_in(f32x4_t (&v)[NV], int nv, float* part, int S,
                                              int s, uint32_t* cnt, int* s_last) {
  const int tid = threadIdx.x;
  float* mine = part + static_cast<size_t>(s) * NV * kThreads * 4;
#pragma unroll
  for (int q = 0; q < NV; ++q)
    if (q < nv)
      st_f32x4<true>(mine + (static_cast<size_t>(q) * kThreads + tid) * 4,
                     make_float4(v[q][0], v[q][1], v[q][2], v[q][3]));
  wait_memory();
  __syncthreads();
  if (tid == 0)
    *s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              static_cast<uint32_t>(S) - 1;
  __syncthreads();
  if (!*s_last) return false;
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // QC slots at a time: at most 16 float4 loads (and their addresses) held
  constexpr int QC = 16 / MAXS < NV ? (16 / MAXS > 0 ? 16 / MAXS : 1) : NV;
  static_assert(NV % QC == 0, "whole chunks of slots");
#pragma unroll
  for (int q0 = 0; q0 < NV; q0 += QC) {
    float4 y[QC][MAXS];
#pragma unroll
    for (int q = 0; q < QC; ++q)
#pragma unroll
      for (int r = 0; r < MAXS; ++r)
      {
        // uniform slot base (scalar registers) + the thread's 16 bytes
        const float* slot = part + (static_cast<size_t>(r < S ? r : s) * NV + q0 + q) * kThreads * 4;
        y[q][r] = *reinterpret_cast<const float4*>(slot + tid * 4);
      }
#pragma unroll
    for (int q = 0; q < QC; ++q) {
      const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
      f32x4_t t = zero;
#pragma unroll
      for (int r = 0; r < MAXS; ++r) {  // selects, no branches: ranges past S add zero
        const f32x4_t x =
            r == s ? v[q0 + q] : f32x4_t{y[q][r].x, y[q][r].y, y[q][r].z, y[q][r].w};
        t += r < S ? x : zero;
      }
      v[q0 + q] = t;
      asm volatile("" : "+v"(v[q0 + q]));  // the sums are done here, before the next
    }                                       // slots' loads (which stay below)
    asm volatile("" ::: "memory");
  }
  return true;
}

// gate_up + clamped SwiGLU of a dense layer: SwiGLU outputs of row tile
// `tile` (64), tokens [16 GR pass, 16 GR (pass + 1)) as GR 16-token groups,
// contraction range s of S; NB blocks per round of loads.  The activation
// blocks are double-buffered, so one barrier per round orders both the
// staging (its loads are in LDS) and the reuse of a buffer (every wave read
// it two rounds before).
template <bool E8, int GR, int NB>
__global__ __launch_bounds__(kThreads, 2) void dense_gate_up_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ sw13,
    const void* __restrict__ sscale13, int H, int Is, int T, int P, int S, Workspace ws,
    float limit) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  int unit, pass;
  xcd_tile_pass(blockIdx.x, P, &unit, &pass);
  if (unit >= (Is / kDenseGuOuts) * S) return;  // uniform over the workgroup
  const int tile = unit / S, s = unit - tile * S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int i0 = tile * kDenseGuOuts + 16 * wave;  // this wave's SwiGLU outputs
  constexpr int SB = 2 * kSubtileBlock;            // 16 gate + 16 up rows of one block
  unsigned char* wst = smem + wave * NB * SB;
  unsigned char* ast = smem + kWaves * NB * SB;    // [2][NB][GR] activation blocks
  const int KB = H / kBlock;
  int b0, nb;
  k_range(s, S, KB, &b0, &nb);
  const int rot = tile % nb;
  // load rows: instructions 0, 1 = gate rows i0 .. i0 + 15, 2, 3 = up rows
  const uint8_t* lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lrow[i] = sw13 + static_cast<size_t>((i < 2 ? i0 : Is + i0 - 16) + 8 * i + (lane >> 3)) * H;
  const size_t sg0 = static_cast<size_t>(i0 / kBlock) * KB;
  const size_t su0 = static_cast<size_t>((Is + i0) / kBlock) * KB;
  const int p0 = pass * 16 * GR;
  const int G = min(GR, (T - p0 + 15) / 16);  // groups holding tokens (uniform)
  const uint16_t* xsrc[GR];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr)
    xsrc[gr] = act_src(hidden + static_cast<size_t>(min(p0 + 16 * gr + act_row(), T - 1)) * H);
  f32x4_t fg[GR], fu[GR];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    fg[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    fu[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = 0, rd = 0; i < nb; i += NB, ++rd) {
    unsigned char* ab = ast + (rd & 1) * NB * GR * kActBlock;
    float sg[NB], su[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int kb = range_block(i + j, b0, nb, rot);
      stage_block<4>(lrow, kb * kBlock, wst + j * SB);
      // every group, also past G (clamped rows): no branch around the staging
#pragma unroll
      for (int gr = 0; gr < GR; ++gr)
        stage_act(xsrc[gr] + kb * kBlock, ab + (j * GR + gr) * kActBlock);
      const float a = load_scale<E8>(sscale13, sg0 + kb);
      const float b = load_scale<E8>(sscale13, su0 + kb);
      sg[j] = i + j < nb ? a : 0.f;
      su[j] = i + j < nb ? b : 0.f;
    }
    wait_memory();    // this thread's staged pieces are in LDS
    __syncthreads();  // and every other thread's
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const unsigned char* st = wst + j * SB;
      f32x4_t pg[GR], pu[GR];
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {
        pg[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pu[gr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint2 hg = staged_half(st, 0, c, m, g), hu = staged_half(st, 1, c, m, g);
        const bf16x8_t wg = fp8x8_to_bf16x8(hg.x, hg.y), wu = fp8x8_to_bf16x8(hu.x, hu.y);
#pragma unroll
        for (int gr = 0; gr < GR; ++gr) {
          if (gr >= G) break;
          const bf16x8_t a = act_frag(ab + (j * GR + gr) * kActBlock, c, m, g);
          pg[gr] = mfma(a, wg, pg[gr]);
          pu[gr] = mfma(a, wu, pu[gr]);
        }
      }
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {
        if (gr >= G) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fg[gr][e] = fmaf(sg[j], pg[gr][e], fg[gr][e]);
          fu[gr][e] = fmaf(su[j], pu[gr][e], fu[gr][e]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
  }
  // lane (g, c) holds tokens p0 + 16 gr + 4 g + e of SwiGLU output i0 + c
  if (S > 1) {
    f32x4_t v[2 * GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      v[2 * gr] = fg[gr];
      v[2 * gr + 1] = fu[gr];
    }
    const size_t u = static_cast<size_t>(tile) * P + pass;
    float* part = ws.act + u * S * (2 * GR) * kThreads * 4;
    if (!dense_hand_in<2 * GR, kDenseGuMaxSplits>(v, 2 * G, part, S, s, ws.rcnt + u * kSyncStride,
                                                  &s_last))
      return;
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      fg[gr] = v[2 * gr];
      fu[gr] = v[2 * gr + 1];
    }
  }
  uint16_t* act_hi = reinterpret_cast<uint16_t*>(ws.act_s);
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    if (gr >= G) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = p0 + 16 * gr + 4 * g + e;
      if (q < T) {
        const float a = clamped_swiglu(fg[gr][e], fu[gr][e], limit);
        const uint16_t hi = bf16_bits(a);
        const uint16_t lo = bf16_bits(a - bf16_to_f32(hi));
        const size_t o = static_cast<size_t>(q) * Is + i0 + c;
        act_hi[o] = hi;
        act_hi[static_cast<size_t>(T) * Is + o] = lo;
      }
    }
  }
}

// gate_up + clamped SwiGLU of a dense layer of at most 16 tokens: SwiGLU
// outputs [i0, i0 + 16) per workgroup, whose four waves take four contiguous
// ranges of the contraction and add their sums in LDS in wave order.  With
// one token group the activations cost at most as many requests as the
// weights, and no workgroup hands sums to another: measured on MI355X
// (H = 4096, I_s = 8192) 16.1 us at one token against 18.6 for the
// shared-activation kernel above, 17.6 against 17.8 at 16 tokens.
// kDenseWavesNb blocks per round of loads.  Measured per layer at 16 tokens
// (one token): one block (eight rounds per wave at H = 4096) 32.3 us (29.8),
// two 33.8 (30.7), four 36.3 (32.6); eight waves per workgroup 34.3 (31.5);
// two 16-output tiles per wave (256 workgroups) 33.3 (32.7).
constexpr int kDenseWavesNb = 1;
template <bool E8>
__global__ __launch_bounds__(kThreads, 2) void dense_gate_up_waves_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ sw13,
    const void* __restrict__ sscale13, int H, int Is, int T, Workspace ws, float limit) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int tile, pass;
  xcd_tile_pass(blockIdx.x, 1, &tile, &pass);
  const int i0 = tile * 16;
  if (i0 >= Is) return;  // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  constexpr int NB = kDenseWavesNb;      // blocks per round of loads
  constexpr int SB = 2 * kSubtileBlock;  // 16 gate + 16 up rows of one block
  unsigned char* stage = smem + wave * NB * SB;
  const int KB = H / kBlock;
  int b0, nb;
  k_range(wave, kWaves, KB, &b0, &nb);
  const int rot = nb > 0 ? tile % nb : 0;
  // load rows: instructions 0, 1 = gate rows i0 .. i0 + 15, 2, 3 = up rows
  const uint8_t* lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lrow[i] = sw13 + static_cast<size_t>((i < 2 ? i0 : Is + i0 - 16) + 8 * i + (lane >> 3)) * H;
  const size_t sg0 = static_cast<size_t>(i0 / kBlock) * KB;
  const size_t su0 = static_cast<size_t>((Is + i0) / kBlock) * KB;
  // lane (g, c): token c (rows past T repeat the last), line by line: load m
  // takes the 16 bytes at 64 m + 16 g of the token's 256-byte block row, so
  // MFMA m covers columns 32 m + 8 g .. + 7, as staged_half on the weights
  const uint16_t* xrow = hidden + static_cast<size_t>(min(c, T - 1)) * H + 8 * g;
  f32x4_t fg = {0.f, 0.f, 0.f, 0.f}, fu = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nb; i += NB) {
    float sg[NB], su[NB];
    int kbs[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int kb = range_block(i + j, b0, nb, rot);
      kbs[j] = kb;
      stage_block<4>(lrow, kb * kBlock, stage + j * SB);
      const float a = load_scale<E8>(sscale13, sg0 + kb);
      const float b = load_scale<E8>(sscale13, su0 + kb);
      sg[j] = i + j < nb ? a : 0.f;
      su[j] = i + j < nb ? b : 0.f;
    }
    asm volatile("" ::: "memory");
    uint4 xa[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xa[j][m] = *reinterpret_cast<const uint4*>(xrow + kbs[j] * kBlock + 32 * m);
    wait_memory();  // the staged weights are in LDS
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const unsigned char* st = stage + j * SB;
      f32x4_t pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint2 hg = staged_half(st, 0, c, m, g), hu = staged_half(st, 1, c, m, g);
        const bf16x8_t a = as_bf16x8(xa[j][m]);
        pg = mfma(a, fp8x8_to_bf16x8(hg.x, hg.y), pg);
        pu = mfma(a, fp8x8_to_bf16x8(hu.x, hu.y), pu);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fg[e] = fmaf(sg[j], pg[e], fg[e]);
        fu[e] = fmaf(su[j], pu[e], fu[e]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): stage reads done
  }
  // The four ranges meet in LDS (the stage is free once every wave is past
  // its last round): lane (g, c) of each wave holds tokens 4 g + e of SwiGLU
  // output i0 + c; wave w then finishes e = w, adding the waves in order.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    red[(wave * 8 + e) * kWave + lane] = fg[e];
    red[(wave * 8 + 4 + e) * kWave + lane] = fu[e];
  }
  __syncthreads();
  const int q = 4 * g + wave;
  if (q < T) {
    float ga = 0.f, ua = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      ga += red[(v * 8 + wave) * kWave + lane];
      ua += red[(v * 8 + 4 + wave) * kWave + lane];
    }
    const float a = clamped_swiglu(ga, ua, limit);
    const uint16_t hi = bf16_bits(a);
    const uint16_t lo = bf16_bits(a - bf16_to_f32(hi));
    uint16_t* act_hi = reinterpret_cast<uint16_t*>(ws.act_s);
    const size_t o = static_cast<size_t>(q) * Is + i0 + c;
    act_hi[o] = hi;
    act_hi[static_cast<size_t>(T) * Is + o] = lo;
  }
}

// down projection of a dense layer: output rows of row tile `rt` (128; wave
// w rows 32 w .. 32 w + 31), tokens [16 GR pass, 16 GR (pass + 1)) as GR
// groups, contraction range s of S, NB blocks per round; the last
// workgroup of the tile writes the rows' sums to ws.y_s [T][H].  The
// activations (the hi and lo planes) are staged as in the gate_up kernel.
template <bool E8, int GR, int NB>
__global__ __launch_bounds__(kThreads, 2) void dense_down_mfma_kernel(
    const uint8_t* __restrict__ sw2, const void* __restrict__ sscale2, int H, int Is, int T,
    int P, int S, Workspace ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  int unit, pass;
  xcd_tile_pass(blockIdx.x, P, &unit, &pass);
  if (unit >= (H / kDenseDnRows) * S) return;  // uniform over the workgroup
  const int rt = unit / S, s = unit - rt * S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int h0 = rt * kDenseDnRows + 32 * wave;  // this wave's rows
  constexpr int SB = 2 * kSubtileBlock;          // 32 rows of one block
  unsigned char* wst = smem + wave * NB * SB;
  unsigned char* ast = smem + kWaves * NB * SB;  // [2][NB][GR][hi, lo] activation blocks
  const int KB = Is / kBlock;
  int b0, nb;
  k_range(s, S, KB, &b0, &nb);
  const int rot = rt % nb;
  const uint8_t* lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lrow[i] = sw2 + static_cast<size_t>(h0 + 8 * i + (lane >> 3)) * Is;
  const size_t s0 = static_cast<size_t>(h0 / kBlock) * KB;
  const int p0 = pass * 16 * GR;
  const int G = min(GR, (T - p0 + 15) / 16);
  const uint16_t* act_hi = reinterpret_cast<const uint16_t*>(ws.act_s);
  const size_t lo_ofs = static_cast<size_t>(T) * Is;
  const uint16_t* asrc[GR];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr)
    asrc[gr] = act_src(act_hi + static_cast<size_t>(min(p0 + 16 * gr + act_row(), T - 1)) * Is);
  f32x4_t f[GR][2];
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    f[gr][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f[gr][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = 0, rd = 0; i < nb; i += NB, ++rd) {
    unsigned char* ab = ast + (rd & 1) * NB * GR * 2 * kActBlock;
    float sc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int kb = range_block(i + j, b0, nb, rot);
      stage_block<4>(lrow, kb * kBlock, wst + j * SB);
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {  // every group (clamped rows), as in gate_up
        unsigned char* blk = ab + (j * GR + gr) * 2 * kActBlock;
        stage_act(asrc[gr] + kb * kBlock, blk);
        stage_act(asrc[gr] + lo_ofs + kb * kBlock, blk + kActBlock);
      }
      const float a = load_scale<E8>(sscale2, s0 + kb);
      sc[j] = i + j < nb ? a : 0.f;
    }
    wait_memory();    // this thread's staged pieces are in LDS
    __syncthreads();  // and every other thread's
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // the block's weight fragments (both 16-row subtiles) once, then each
      // group's activation fragments, each feeding both subtiles
      bf16x8_t wa[2][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint2 hw = staged_half(wst + j * SB, sub, c, m, g);
          wa[sub][m] = fp8x8_to_bf16x8(hw.x, hw.y);
        }
#pragma unroll
      for (int gr = 0; gr < GR; ++gr) {
        if (gr >= G) break;
        const unsigned char* blk = ab + (j * GR + gr) * 2 * kActBlock;
        f32x4_t p[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8_t ah = act_frag(blk, c, m, g);
          const bf16x8_t al = act_frag(blk + kActBlock, c, m, g);
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            p[sub] = mfma(ah, wa[sub][m], p[sub]);
            p[sub] = mfma(al, wa[sub][m], p[sub]);
          }
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int e = 0; e < 4; ++e) f[gr][sub][e] = fmaf(sc[j], p[sub][e], f[gr][sub][e]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
  }
  // lane (g, c) holds tokens p0 + 16 gr + 4 g + e of rows h0 + 16 sub + c
  if (S > 1) {
    f32x4_t v[2 * GR];
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      v[2 * gr] = f[gr][0];
      v[2 * gr + 1] = f[gr][1];
    }
    const size_t u = static_cast<size_t>(rt) * P + pass;
    float* part = ws.act + u * S * (2 * GR) * kThreads * 4;
    if (!dense_hand_in<2 * GR, kDenseDnMaxSplits>(v, 2 * G, part, S, s, ws.rcnt + u * kSyncStride,
                                                  &s_last))
      return;
#pragma unroll
    for (int gr = 0; gr < GR; ++gr) {
      f[gr][0] = v[2 * gr];
      f[gr][1] = v[2 * gr + 1];
    }
  }
#pragma unroll
  for (int gr = 0; gr < GR; ++gr) {
    if (gr >= G) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = p0 + 16 * gr + 4 * g + e;
      if (q < T) {
        float* out = ws.y_s + static_cast<size_t>(q) * H + h0 + c;
        out[0] = f[gr][0][e];
        out[16] = f[gr][1][e];
      }
    }
  }
}

// grid rows: the shared expert's passes, then the touched-expert slots
int shared_rows(const LayerDims& d, int gr = kGR) {
  return d.Is > 0 ? (d.T + 16 * gr - 1) / (16 * gr) : 0;
}
int slot_rows(const LayerDims& d) { return d.T * d.k < d.E ? d.T * d.k : d.E; }

}  // namespace

hipError_t launch_gate_up_mfma(const LayerDims& d, int rows, const void* hidden, const void* w13,
                               const void* w13_scale, const void* sw13, const void* sw13_scale,
                               const Workspace& ws, hipStream_t s, hipEvent_t evb,
                               hipEvent_t eve) {
  const int SP = rows == kRoutedRows ? 0 : shared_rows(d, rows == kSharedRows ? shared_gr(d) : kGR);
  const int R = rows == kSharedRows ? 0 : slot_rows(d);
  if (SP + R == 0) return hipSuccess;
  const int Imax = d.I > d.Is ? d.I : d.Is;
  const int per_wg = kWaves * 8 * kNsGu;  // SwiGLU outputs per workgroup
  dim3 grid((Imax + per_wg - 1) / per_wg, SP + R);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint8_t*>(w13);
  const auto* sw = static_cast<const uint8_t*>(sw13);
#define MOE_GU(E8, ROWS, GR, SA) \
  launch_gu<E8, ROWS, GR, kNsGu, SA>(grid, s, x, w, w13_scale, sw, sw13_scale, d, SP, ws, evb, eve)
  // two groups with shared tiles: waves of kNsGuWide subtiles where they
  // divide I (every wave of a workgroup must meet its barriers)
  const int per_wg_w = kWaves * 8 * kNsGuWide;
  const dim3 grid_w((d.I + per_wg_w - 1) / per_wg_w, SP + R);
  const bool wide = rows == kRoutedRows && d.I % per_wg_w == 0;
#define MOE_GU_WIDE(E8)                                                                   \
  launch_gu<E8, kRoutedRows, 2, kNsGuWide, true>(grid_w, s, x, w, w13_scale, sw, sw13_scale, d, \
                                                 SP, ws, evb, eve)
  if (rows == kAllRows) {
    if (d.e8m0) MOE_GU(true, kAllRows, kGR, false); else MOE_GU(false, kAllRows, kGR, false);
  } else if (rows == kSharedRows && shared_gr(d) == 2) {
    if (d.e8m0) MOE_GU(true, kSharedRows, 2, true); else MOE_GU(false, kSharedRows, 2, true);
  } else if (rows == kSharedRows) {
    if (d.e8m0) MOE_GU(true, kSharedRows, kGR, false); else MOE_GU(false, kSharedRows, kGR, false);
  } else if (routed_gr2(d)) {
    // the shared tiles need the larger mean (kSharedActMinMean >= kGr2MinMean)
    if (routed_sa(d) && wide) {
      if (d.e8m0) MOE_GU_WIDE(true); else MOE_GU_WIDE(false);
    } else if (routed_sa(d)) {
      if (d.e8m0) MOE_GU(true, kRoutedRows, 2, true); else MOE_GU(false, kRoutedRows, 2, true);
    } else {
      if (d.e8m0) MOE_GU(true, kRoutedRows, 2, false); else MOE_GU(false, kRoutedRows, 2, false);
    }
  } else if (routed_sa1(d)) {
    if (d.e8m0) MOE_GU(true, kRoutedRows, kGR, true); else MOE_GU(false, kRoutedRows, kGR, true);
  } else {
    if (d.e8m0) MOE_GU(true, kRoutedRows, kGR, false);
    else MOE_GU(false, kRoutedRows, kGR, false);
  }
#undef MOE_GU
#undef MOE_GU_WIDE
  return hipGetLastError();
}

// Token groups, passes and contraction ranges of a dense layer's launches.
// The down kernel takes at most kDenseDnMaxGroups groups per workgroup: with
// four, its activation blocks (two rounds, hi and lo planes) would not leave
// room for two workgroups per CU.
constexpr int kDenseDnMaxGroups = 2;
struct DenseGrid {
  int gr_gu, p_gu, n_gu, s_gu;  // gate_up: groups per workgroup, passes, row tiles, ranges
  int gr_dn, p_dn, n_dn, s_dn;  // down
};
static int dense_gr(int groups, int max_gr) {
  const int gr = groups >= 4 ? 4 : (groups >= 2 ? 2 : 1);
  return gr < max_gr ? gr : max_gr;
}
static DenseGrid dense_grid(int T, int H, int Is) {
  DenseGrid g;
  const int groups = (T + 15) / 16;
  g.gr_gu = dense_gr(groups, kDenseMaxGroups);
  g.p_gu = (groups + g.gr_gu - 1) / g.gr_gu;
  g.n_gu = Is / kDenseGuOuts;
  // (one group: dense_gate_up_waves_mfma_kernel, no ranges to hand over)
  g.s_gu = groups == 1 ? 1 : dense_splits(g.n_gu, g.p_gu, H / kBlock, kDenseGuMaxSplits);
  g.gr_dn = dense_gr(groups, kDenseDnMaxGroups);
  g.p_dn = (groups + g.gr_dn - 1) / g.gr_dn;
  g.n_dn = H / kDenseDnRows;
  g.s_dn = dense_splits(g.n_dn, g.p_dn, Is / kBlock, kDenseDnMaxSplits);
  return g;
}

// (the grid depends on the token count only through its 16-token groups)
size_t dense_part_floats(int maxT, int H, int Is) {
  if (maxT < 1 || H < kDenseDnRows || Is < kDenseGuOuts) return 0;
  size_t most = 0;
  for (int groups = 1; groups <= (maxT + 15) / 16; ++groups) {
    const DenseGrid g = dense_grid(16 * groups, H, Is);
    const size_t gu = g.s_gu > 1 ? static_cast<size_t>(2 * g.gr_gu) * kThreads * 4 * g.p_gu *
                                       g.n_gu * g.s_gu
                                 : 0;
    const size_t dn = g.s_dn > 1 ? static_cast<size_t>(2 * g.gr_dn) * kThreads * 4 * g.p_dn *
                                       g.n_dn * g.s_dn
                                 : 0;
    most = std::max(most, std::max(gu, dn));
  }
  return most;
}

int dense_count_lines(int maxT, int H, int Is) {
  if (maxT < 1 || H < kDenseDnRows || Is < kDenseGuOuts) return 0;
  return std::max(Is / kDenseGuOuts, H / kDenseDnRows) * ((maxT + 15) / 16);
}

template <bool E8, int GR>
static void launch_dense_gate_up(const LayerDims& d, const DenseGrid& g, const uint16_t* x,
                                 const uint8_t* w13, const void* s13, const Workspace& ws,
                                 hipStream_t s, hipEvent_t evb, hipEvent_t eve) {
  constexpr int NB = GR == kDenseMaxGroups ? 1 : 2;  // blocks per round
  const size_t lds = kWaves * NB * 2 * kSubtileBlock + 2 * NB * GR * static_cast<size_t>(kActBlock);
  const int units = g.n_gu * g.s_gu;
  const dim3 grid(static_cast<unsigned>((units + kXcds - 1) / kXcds * kXcds * g.p_gu));
  MOE_LAUNCH((dense_gate_up_mfma_kernel<E8, GR, NB>), grid, dim3(kThreads), lds, s, evb, eve, x,
             w13, s13, d.H, d.Is, d.T, g.p_gu, g.s_gu, ws, d.limit);
}

template <bool E8>
static void launch_dense_gate_up_waves(const LayerDims& d, const uint16_t* x, const uint8_t* w13,
                                       const void* s13, const Workspace& ws, hipStream_t s,
                                       hipEvent_t evb, hipEvent_t eve) {
  // the stage, or the waves' sums after it (4 waves x 8 x 64 floats)
  const size_t lds =
      std::max<size_t>(kWaves * kDenseWavesNb * 2 * kSubtileBlock, kWaves * 8 * kWave * 4);
  const int units = d.Is / 16;
  const dim3 grid(static_cast<unsigned>((units + kXcds - 1) / kXcds * kXcds));
  MOE_LAUNCH((dense_gate_up_waves_mfma_kernel<E8>), grid, dim3(kThreads), lds, s, evb, eve, x,
             w13, s13, d.H, d.Is, d.T, ws, d.limit);
}

template <bool E8, int GR>
static void launch_dense_down(const LayerDims& d, const DenseGrid& g, const uint8_t* w2,
                              const void* s2, const Workspace& ws, hipStream_t s) {
  // blocks per round: four for one group (one workgroup per CU at 16 tokens:
  // 33.9 us per layer against 34.7 with two, one token 30.7 against 31.3),
  // one for two groups (LDS for two workgroups per CU)
  constexpr int NB = GR == 1 ? 4 : 1;
  const size_t lds = kWaves * NB * 2 * kSubtileBlock +
                     2 * NB * 2 * GR * static_cast<size_t>(kActBlock);
  const int units = g.n_dn * g.s_dn;
  const dim3 grid(static_cast<unsigned>((units + kXcds - 1) / kXcds * kXcds * g.p_dn));
  hipLaunchKernelGGL((dense_down_mfma_kernel<E8, GR, NB>), grid, dim3(kThreads), lds, s, w2, s2,
                     d.H, d.Is, d.T, g.p_dn, g.s_dn, ws);
}

hipError_t launch_dense_mfma(const LayerDims& d, const void* hidden, const void* sw13,
                             const void* sw13_scale, const void* sw2, const void* sw2_scale,
                             const Workspace& ws, hipStream_t s, hipEvent_t evb, hipEvent_t eve) {
  if (d.E != 0 || d.Is <= 0 || d.T <= 0 || d.H % kDenseDnRows || d.Is % kDenseGuOuts)
    return hipErrorInvalidValue;
  const DenseGrid g = dense_grid(d.T, d.H, d.Is);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w13 = static_cast<const uint8_t*>(sw13);
  const auto* w2 = static_cast<const uint8_t*>(sw2);
#define MOE_GU(E8, GR_) launch_dense_gate_up<E8, GR_>(d, g, x, w13, sw13_scale, ws, s, evb, eve)
  if (g.gr_gu == 1) {  // one token group: the waves split the contraction
    if (d.e8m0) launch_dense_gate_up_waves<true>(d, x, w13, sw13_scale, ws, s, evb, eve);
    else launch_dense_gate_up_waves<false>(d, x, w13, sw13_scale, ws, s, evb, eve);
  } else if (g.gr_gu == 2) {
    if (d.e8m0) MOE_GU(true, 2); else MOE_GU(false, 2);
  } else {
    if (d.e8m0) MOE_GU(true, kDenseMaxGroups); else MOE_GU(false, kDenseMaxGroups);
  }
#undef MOE_GU
#define MOE_DN(E8, GR_) launch_dense_down<E8, GR_>(d, g, w2, sw2_scale, ws, s)
  if (g.gr_dn == 1) {
    if (d.e8m0) MOE_DN(true, 1); else MOE_DN(false, 1);
  } else {
    if (d.e8m0) MOE_DN(true, kDenseDnMaxGroups); else MOE_DN(false, kDenseDnMaxGroups);
  }
#undef MOE_DN
  return hipGetLastError();
}

hipError_t launch_down_mfma(const LayerDims& d, int rows, const void* w2, const void* w2_scale,
                            const void* sw2, const void* sw2_scale, const Workspace& ws,
                            hipStream_t s) {
  const int SP = rows == kRoutedRows ? 0 : shared_rows(d, rows == kSharedRows ? shared_gr(d) : kGR);
  const int R = rows == kSharedRows ? 0 : slot_rows(d);
  if (SP + R == 0) return hipSuccess;
  const auto* w = static_cast<const uint8_t*>(w2);
  const auto* sw = static_cast<const uint8_t*>(sw2);
#define MOE_DN(NS, E8, ROWS, GR, SA) \
  launch_dn<NS, E8, ROWS, GR, SA>(R, s, w, w2_scale, sw, sw2_scale, d, SP, ws)
  if (rows == kAllRows) {
    if (d.e8m0) MOE_DN(kNsDn, true, kAllRows, kGR, false);
    else MOE_DN(kNsDn, false, kAllRows, kGR, false);
  } else if (rows == kSharedRows && shared_gr(d) == 2) {
    if (d.e8m0) MOE_DN(kNsDn, true, kSharedRows, 2, true);
    else MOE_DN(kNsDn, false, kSharedRows, 2, true);
  } else if (rows == kSharedRows) {
    if (d.e8m0) MOE_DN(kNsDn, true, kSharedRows, kGR, false);
    else MOE_DN(kNsDn, false, kSharedRows, kGR, false);
  } else if (routed_gr2(d) && routed_sa(d)) {
    if (d.e8m0) MOE_DN(kNsDnRouted, true, kRoutedRows, 2, true);
    else MOE_DN(kNsDnRouted, false, kRoutedRows, 2, true);
  } else if (routed_gr2(d)) {
    if (d.e8m0) MOE_DN(kNsDnRouted, true, kRoutedRows, 2, false);
    else MOE_DN(kNsDnRouted, false, kRoutedRows, 2, false);
  } else if (!routed_gr2(d) && routed_sa1(d)) {
    if (d.e8m0) MOE_DN(kNsDnRouted, true, kRoutedRows, kGR, true);
    else MOE_DN(kNsDnRouted, false, kRoutedRows, kGR, true);
  } else {
    if (d.e8m0) MOE_DN(kNsDnRouted, true, kRoutedRows, kGR, false);
    else MOE_DN(kNsDnRouted, false, kRoutedRows, kGR, false);
  }
#undef MOE_DN
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

bool grouped_boundary_fused(const LayerDims& d) { return d.T <= kFusedBoundaryMaxTokens; }

bool grouped_chain_supported(const LayerDims& d) {
  // whole down tiles (every wave of a tile reaches the wait) and whole
  // gate_up tiles; the shared passes fit the flag lines
  static_assert(kThreads == kBndThreads, "the boundary slices are workgroups of this launch");
  return d.T <= kMergeSharedMaxTokens && d.H % (kWaves * 16 * kNsDn) == 0 &&
         (d.H + kBndCols - 1) / kBndCols <= kMaxBndSlices &&
         d.I % (kWaves * 8 * kNsGu) == 0 && d.Is % (kWaves * 8 * kNsGu) == 0 &&
         kNsDn * kWaves * 16 == 256 && shared_rows(d) <= kSyncSlot0 - kSyncFlags &&
         kLdsGu == static_cast<size_t>(kWaves) * kUDn * kNsDn * kSubtileBlock;
}

hipError_t launch_grouped_chain(const LayerDims& d, const void* hidden, const void* w13,
                                const void* w13_scale, const void* sw13, const void* sw13_scale,
                                const void* w2, const void* w2_scale, const void* sw2,
                                const void* sw2_scale, const void* residual, const void* gamma,
                                void* out, void* residual_out, void* moe_out,
                                const Workspace& ws, hipStream_t s, hipEvent_t evb,
                                hipEvent_t eve) {
  if (!grouped_chain_supported(d)) return hipErrorInvalidValue;
  GChainArgs a{};
  a.hidden = static_cast<const uint16_t*>(hidden);
  a.w13 = static_cast<const uint8_t*>(w13);
  a.w13_scale = w13_scale;
  a.sw13 = static_cast<const uint8_t*>(sw13);
  a.sw13_scale = sw13_scale;
  a.w2 = static_cast<const uint8_t*>(w2);
  a.w2_scale = w2_scale;
  a.sw2 = static_cast<const uint8_t*>(sw2);
  a.sw2_scale = sw2_scale;
  a.residual = static_cast<const uint16_t*>(residual);
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.out = static_cast<uint16_t*>(out);
  a.residual_out = static_cast<uint16_t*>(residual_out);
  a.moe_out = static_cast<uint16_t*>(moe_out);
  a.H = d.H;
  a.I = d.I;
  a.Is = d.Is;
  a.k = d.k;
  a.T = d.T;
  a.SP = shared_rows(d);
  a.limit = d.limit;
  a.eps = d.eps;
  const int rows = a.SP + slot_rows(d);
  const int Imax = d.I > d.Is ? d.I : d.Is;
  a.gx = Imax / (kWaves * 8 * kNsGu);
  a.dx = d.H / (kWaves * 16 * kNsDn);
  a.n_gu = a.gx * rows;
  a.n_dn = a.dx * rows;
  const bool bnd = grouped_boundary_fused(d);
  a.bnd_ns = bnd ? (d.H + kBndCols - 1) / kBndCols : 0;
  const int n = a.n_gu + a.n_dn + d.T * a.bnd_ns;
  if (d.e8m0)
    MOE_LAUNCH((grouped_chain_kernel<true>), dim3(n), dim3(kThreads), kLdsGu, s, evb, eve, a, ws);
  else
    MOE_LAUNCH((grouped_chain_kernel<false>), dim3(n), dim3(kThreads), kLdsGu, s, evb, eve, a,
               ws);
  return hipGetLastError();
}

}  // namespace moe
