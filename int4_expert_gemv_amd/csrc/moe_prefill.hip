// moe_prefill.hip -- routed expert FFN for many tokens at once (prefill):
// the expert-grouped batch-union on the MFMA matrix cores.
//
// The colibri page "Vulkan backend: expert tier + dense + MLA attention on
// any Vulkan 1.2 GPU" (PR summary and the pp512 notes) describes prefill as
// expert-streaming-bound: a 512-token batch touches nearly every expert, so
// each routed expert's weights should be read once for all of the tokens
// routed to it.  The pages keep prefill on the CPU; here it is a grouped GEMM:
// the tokens routed to one expert form the M dimension, the expert's output
// features the N dimension.
//
// Arithmetic.  int4 weights become exact integer-valued bf16 operands with
// the same bit trick as the decode kernels: (w >> 4i) & 0x000F000F | 0x43004300
// is the bf16 pair (128 + n_i, 128 + n_{i+4}).  One 32-bit weight word (eight
// consecutive K of one output column) is therefore the B operand of one
// v_mfma_f32_32x32x16_bf16 lane, in the K order n0 n4 n1 n5 n2 n6 n3 n7; the
// activations are stored once in that same pair-permuted order.  The offset
// (128 + 8 = 136 per weight) and the fp32 scale of every K group are applied
// per group: each group's MFMA chain is folded into the accumulator with one
// FMA by the column's scale, and the offset term scale[n][g] * (-136 * sum of
// group g of row m) is a rank-2 update per stage -- one fp32
// v_mfma_f32_32x32x2_f32 over the (at most two) groups that end in the stage,
// so no VALU work per element goes to it.  Activations are bf16 (fp32 input is rounded
// to nearest even) and the hidden vector h = silu(gate x) * up x is rounded to
// bf16 before the down projection -- the prefill precision the oracle models.
//
// Five launches on one stream, no host synchronisation:
//  1. prep     block 0 buckets the T*k (token, slot) pairs by expert: counts,
//              offsets, the list of 32-row M-tiles, pairs sorted by expert;
//              blocks 1..T write each token's x as permuted bf16 plus its
//              per-group sums;
//  2. gate+up  per (M-tile, 256 columns of I): h in sorted-pair order, bf16,
//              plus 32-column sums of h;
//  3. hsum     per-group sums of h for the down projection;
//  4. down     per (M-tile, 512 columns of H): per-pair outputs, fp32;
//  5. combine  y[t] = sum over slots j, in order, of w[t][j] * out[t*k+j].
// Every output element is a fixed-order sum that does not depend on where its
// pair lands inside a tile, so y is identical from run to run even though the
// bucketing uses atomics.
#include "device.hpp"
#include "launch.hpp"
#include "qmoe.h"

namespace qm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define QM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kBM = 32;         // tokens per M-tile (one 32-row MFMA subtile)
constexpr int kBK = 256;        // K per pipeline stage: a 128-byte line of every weight row
#ifndef QM_PF_STAGES
#define QM_PF_STAGES 3
#endif
constexpr int kGW = 16;         // waves per GEMM workgroup
constexpr int kGT = 64 * kGW;   // threads per GEMM workgroup
constexpr int kStages = QM_PF_STAGES;  // LDS ring depth
constexpr int kEMax = 8192;     // experts the bucketing block handles in LDS

struct Tile {
  int e, m0, mrows, pos0;  // expert, first row within the expert, valid rows, first sorted position
};

struct PrepArgs {
  const void* x;         // [T][H] fp32 or bf16
  const int32_t* ids;    // [T][k]
  int T, topk, E, H;
  int G, nb32;           // groups per row of H and 32-element blocks per group
  int* hdr;              // [0] = number of M-tiles
  int* off;              // [E + 1] start of each expert's pairs in `sorted`
  Tile* tiles;           // [mt_max]
  int* sorted;           // [T*k] pair indices grouped by expert
  uint16_t* xp;          // [T][H] bf16, pair-permuted within every 8 elements
  float* xsg;            // [T][G] group sums of the bf16 x
};

template <int NM>
struct GemmArgs {
  const uint8_t* wq[NM];  // stacked expert weights: gate, up (NM = 2) or down (NM = 1)
  const float* wsc[NM];   // their scales
  int64_t rb;             // bytes per weight row (K / 2)
  int64_t eq, es;         // per-expert stride of the weights (bytes) and scales (floats)
  int N, K;               // output features and reduction length
  int G, gs_ch, gs_sh;    // scale groups per row, 64-K chunks per group (a power of two when G > 1) and its log2
  const int* hdr;
  const Tile* tiles;
  const int* sorted;
  const uint16_t* a;      // A rows (bf16, permuted): xp by token (gate+up) or h by sorted position (down)
  const float* asum;      // [A row][G] group sums of the A rows
  int topk;               // gate+up: A row = sorted[pos] / topk; down: A row = pos
  int mt_max, nt;
  uint16_t* h;            // gate+up: h [P][N] bf16 permuted, sorted order
  float* h32;             // gate+up: [P][N / 32] sums of 32 consecutive h
  float* out;             // down: [T*k][N] per-pair outputs
};

// ---- 1. prep ---------------------------------------------------------------------

__device__ void bucket_pairs(const PrepArgs& a, int* sh) {
  const int tid = threadIdx.x, E = a.E, P = a.T * a.topk;
  int* cnt = sh;             // [E] counts, then cursors
  int* s_a = sh + E;         // [256] per-thread sums of counts
  int* s_b = s_a + kThreads; // [256] per-thread sums of tile counts
  for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int id = a.ids[p];
    if (id >= 0 && id < E) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sa = 0, sb = 0;
  for (int e = e0; e < e1; ++e) {
    sa += cnt[e];
    sb += (cnt[e] + kBM - 1) / kBM;
  }
  s_a[tid] = sa;
  s_b[tid] = sb;
  __syncthreads();
  if (tid == 0) {
    int ra = 0, rb = 0;
    for (int i = 0; i < kThreads; ++i) {
      const int va = s_a[i], vb = s_b[i];
      s_a[i] = ra;
      s_b[i] = rb;
      ra += va;
      rb += vb;
    }
    a.off[E] = ra;
    a.hdr[0] = rb;
  }
  __syncthreads();
  int pos = s_a[tid], tile = s_b[tid];
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    a.off[e] = pos;
    for (int m0 = 0; m0 < c; m0 += kBM) a.tiles[tile++] = Tile{e, m0, min(kBM, c - m0), pos + m0};
    cnt[e] = pos;
    pos += c;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int id = a.ids[p];
    if (id >= 0 && id < E) a.sorted[atomicAdd(&cnt[id], 1)] = p;
  }
}

template <int XT>
__device__ void permute_token(const PrepArgs& a, int t, float* s32) {
  const int nblk = a.H / 32;
  for (int b = threadIdx.x; b < nblk; b += kThreads) {
    uint32_t v[32];  // bf16 bits of x[t][32b + i]
    if constexpr (XT == kBF16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * a.H + 32 * b);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w = src[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * q + 2 * i] = w[i] & 0xFFFFu;
          v[8 * q + 2 * i + 1] = w[i] >> 16;
        }
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + (int64_t)t * a.H + 32 * b);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 f = src[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * q + i] = f32_to_bf16_bits(f[i]);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += bf16_bits_to_f32(v[i]);
    u32x4* dst = reinterpret_cast<u32x4*>(a.xp + (int64_t)t * a.H + 32 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = v[8 * q + i] | (v[8 * q + 4 + i] << 16);
      dst[q] = o;
    }
    s32[b] = s;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < a.G; g += kThreads) {
    float s = 0.f;
    for (int i = 0; i < a.nb32; ++i) s += s32[g * a.nb32 + i];
    a.xsg[(int64_t)t * a.G + g] = s;
  }
}

template <int XT>
__global__ __launch_bounds__(kThreads) void prefill_prep_kernel(PrepArgs a) {
  extern __shared__ __attribute__((aligned(16))) int sh[];
  if (blockIdx.x == 0)
    bucket_pairs(a, sh);
  else
    permute_token<XT>(a, blockIdx.x - 1, reinterpret_cast<float*>(sh));
}

// ---- 2./4. grouped GEMM on MFMA -----------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | (((N >> 4) & 3) << 14));
}

// Workgroup barrier for the LDS ring.  __syncthreads() carries a release
// fence, for which the compiler waits for every outstanding memory operation
// (vmcnt(0)), draining the DMA stages that should stay in flight.  Here only
// this wave's LDS operations are waited for; the DMA of the stage about to be
// read was waited for explicitly, and the empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int rotated(int it, int rot, int n) {
  const int v = it + rot;
  return v < n ? v : v - n;
}

// The B operand is built in plain C so that the compiler sees every VALU
// write feeding the MFMA and inserts the required wait states (an inline-asm
// producer is opaque to its hazard tracking).  `base` is the bf16 pair
// 128.0|128.0 held in a VGPR, so (v & mask) | base selects v_and_or_b32
// (mask in an SGPR): 7 VALU operations per 8 weights.
__device__ __forceinline__ bf16x8 b_operand(uint32_t w, uint32_t base) {
  u32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = ((w >> (4 * i)) & 0x000F000Fu) | base;
  return __builtin_bit_cast(bf16x8, p);
}

// Block: 16 waves over one M-tile of BM = 32 rows (tokens) and 256 weight
// rows.  Waves w and w + 8 own the same 32-column tile of weight rows
// [32 (w & 7), 32 (w & 7) + 32) and split every stage's 256 K: wave w the
// first 128 (chunks 0, 1), wave w + 8 the second (chunks 2, 3); their two
// partial tiles are added in the epilogue.  For gate+up (NM = 2) tiles 0-3
// are gate columns and tiles 4-7 the up columns of the same 128 outputs, for
// down (NM = 1) the 256 outputs.  Four waves per SIMD keep the matrix cores,
// the VALU work that builds B operands and folds groups, and the LDS reads
// of different waves overlapping.
//
// A stage reads a whole 128-byte line of every weight row (K = 256), so each
// line is fetched into L2 once: with half a line per stage the other half
// was needed a stage later, by when the line had often been evicted by the
// other workgroups' streams and came from HBM a second time.  Per stage the
// block DMAs into one LDS ring slot:
//   A   BM rows x 512 B, piece p of row r at slot p ^ (r & 15)
//   B   256 weight rows x 128 B, piece p of row rr at slot p ^ ((rr >> 1) & 7)
//   SC  (grouped scales) per weight row the aligned 16 bytes holding the
//       scales of the stage's groups
//   CR  (grouped scales) per A row the aligned 16 bytes holding the sums of
//       the stage's groups, for the offset correction
// so that the ds_read_b128 operand reads of 16 consecutive lanes hit distinct
// banks.  Every wave issues four DMA operations per stage -- one A piece, two
// B pieces, and one of the 288 SC/CR pieces (18 lanes each) -- which is what
// its vmcnt waits count; two stages stay in flight while one is used.  With
// one scale per row (ROWSC) a lane keeps its column's scale in a register, no
// scales move and the correction sums are a 32-entry table.
template <int NM, bool ROWSC_>
struct GemmShape {
  static constexpr bool ROWSC = ROWSC_;
  static constexpr int BM = kBM;
  static constexpr int ROWS = kGW / 2 * 32;  // weight rows of a block
  static constexpr int BN = ROWS / NM;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * kBK * 2;
  static constexpr int SC_OFF = B_OFF + ROWS * kBK / 2;
  static constexpr int CR_OFF = SC_OFF + ROWS * 16;
  static constexpr int SLOT = ROWSC ? SC_OFF : CR_OFF + BM * 16;  // one ring stage
  static constexpr int CORR_OFF = kStages * SLOT;                  // ROWSC: the 32 correction values
  static constexpr int LDS = CORR_OFF + (ROWSC ? BM * 4 : 0);
  static constexpr int XCH = kGW / 2 * 16 * 64 * 4;               // epilogue exchange (reuses the ring)
  static constexpr int XP = ROWSC ? 0 : (ROWS + BM + kGW - 1) / kGW;  // SC/CR pieces per wave
  static_assert(BM * 32 == kGT && ROWS * 8 == 2 * kGT, "piece split");
  static_assert(LDS + 2 * BM * 4 <= 160 * 1024 && XCH <= LDS, "LDS budget");
};

template <int NM, typename T>
__device__ __forceinline__ T pick(T const (&v)[NM], int m) {
  return NM == 1 || m == 0 ? v[0] : v[NM - 1];
}

// The four DMA operations of a wave for one pipeline stage into LDS slot
// `slot`.  Every source address is fixed per thread except for the stage's
// K offset (A: 512 bytes, B: 128 bytes, SC/CR: one 16-byte piece).
struct StageSrc {
  const uint16_t* arow;    // this thread's A row, its piece offset in elements
  int apc;
  const uint8_t* brow[2];  // its two B rows, piece offsets in bytes
  int bpc[2];
  const float* xrow;       // its SC or CR row (grouped scales), null for none
};

template <typename S>
__device__ __forceinline__ void issue_stage(char* lds, int st, int slot, int wave, int lane, int gs_sh,
                                            const StageSrc& src) {
  char* sd = lds + slot * S::SLOT;
  __builtin_amdgcn_global_load_lds(src.arow + st * kBK + src.apc, QM_LDS_PTR(sd + S::A_OFF + wave * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(src.brow[i] + st * (kBK / 2) + src.bpc[i],
                                     QM_LDS_PTR(sd + S::B_OFF + (i * kGW + wave) * 1024), 16, 0, 0);
  if constexpr (!S::ROWSC) {
    // the aligned four groups holding the stage's first group
    const int piece = ((st * 4) >> gs_sh) >> 2;
    if (lane < S::XP)
      __builtin_amdgcn_global_load_lds(src.xrow + 4 * piece, QM_LDS_PTR(sd + S::SC_OFF + wave * S::XP * 16), 16, 0, 0);
  }
}

// GM, the scale grouping the loop is compiled for: 0 one scale per row,
// 1 groups of 64 K (every chunk starts and ends a group), 2 groups of 128 K
// or more (a wave's two chunks of a stage lie in one group).  Where a chunk
// starts a group at compile time its first MFMA takes the inline constant 0
// as C.
template <int NM, int GM>
__global__ __launch_bounds__(kGT) void prefill_gemm_kernel(GemmArgs<NM> a) {
  constexpr bool ROWSC = GM == 0;
  using S = GemmShape<NM, ROWSC>;
  constexpr int HW = kGW / 2;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_row[S::BM];   // A row index of each tile row
  __shared__ int s_pair[S::BM];  // pair index of each tile row
  const int nb = gridDim.x;
  const int L = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);  // consecutive tiles share an XCD
  const int mt = L % a.mt_max, nti = L / a.mt_max;
  if (nti >= a.nt || mt >= a.hdr[0]) return;
  const Tile tl = a.tiles[mt];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = nti * S::BN;
  if (tid < S::BM) {
    const int r = tid < tl.mrows ? tid : 0;
    const int p = a.sorted[tl.pos0 + r];
    s_pair[tid] = p;
    s_row[tid] = NM == 2 ? p / a.topk : tl.pos0 + r;
  }
  __syncthreads();

  const int nstages = a.K / kBK;
  const int h = lane >> 5, c32 = lane & 31;
  const int kh = wave / HW, wl = wave % HW;  // K half of the stage, column tile
  const int mat = wl / (HW / NM);            // this wave's matrix
  const int rw = wl * 32 + c32;              // its weight row within the block
  // one scale per row: this lane's column, and the correction values of the
  // A rows (-136 * the row's sum)
  const float rsc = ROWSC ? pick(a.wsc, mat)[(int64_t)tl.e * a.es + n0 + (wl % (HW / NM)) * 32 + c32] : 0.f;
  float* corr0 = reinterpret_cast<float*>(lds + S::CORR_OFF);
  if (ROWSC && tid < S::BM) corr0[tid] = -136.f * a.asum[s_row[tid]];
  // per-thread DMA sources (rows fixed for the whole K loop)
  StageSrc src;
  {
    const int P = wave * 64 + lane;  // A piece: row P >> 5, slot P & 31
    const int r = P >> 5;
    src.arow = a.a + (int64_t)s_row[r] * a.K;
    src.apc = 8 * ((P & 31) ^ (r & 15));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = (i * kGW + wave) * 64 + lane;  // B piece: row P >> 3, slot P & 7
    const int rr = P >> 3;
    src.brow[i] = pick(a.wq, rr / S::BN) + (int64_t)tl.e * a.eq + (int64_t)(n0 + rr % S::BN) * a.rb;
    src.bpc[i] = 16 * ((P & 7) ^ ((rr >> 1) & 7));
  }
  src.xrow = nullptr;
  if constexpr (!ROWSC) {
    const int X = wave * S::XP + (lane < S::XP ? lane : 0);  // SC piece X < ROWS, then CR pieces
    if (X < S::ROWS)
      src.xrow = pick(a.wsc, X / S::BN) + (int64_t)tl.e * a.es + (int64_t)(n0 + X % S::BN) * a.G;
    else
      src.xrow = a.asum + (int64_t)s_row[min(X - S::ROWS, S::BM - 1)] * a.G;
  }
  // Blocks walk K from different stages: weight rows lie a multiple of
  // 1 KiB apart, so blocks that all stood at the same K offset would all hit
  // the same few L2 channels.  The rotation depends on the expert and the
  // column tile only, never on which M-tile a pair landed in (the bucketing
  // order is not fixed), so every output keeps one summation order from run
  // to run.
  const int rot = (tl.e * 7 + nti * 3) % nstages;
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < nstages) issue_stage<S>(lds, rotated(i, rot, nstages), i, wave, lane, a.gs_sh, src);

  uint32_t base = 0x43004300u;
  asm volatile("" : "+v"(base));  // keep the constant in a VGPR (see b_operand)
  f32x16 acc = {}, tmp = {};
  for (int it = 0; it < nstages; ++it) {
    // the wave's DMA operations of stage it + 1 (four; three without scales)
    // may stay in flight
    static_assert(kStages == 3, "the waits below count one stage in flight");
    if (it + 1 < nstages)
      wait_vm<ROWSC ? 3 : 4>();
    else
      wait_vm<0>();
    ring_barrier();  // this stage is in LDS for every wave; the previous one's slot is free
    const char* sd = lds + (it % kStages) * S::SLOT;
    const int st = rotated(it, rot, nstages);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = st * 4 + 2 * kh + c;  // 64-K chunk of the row
      const int g = chunk >> a.gs_sh;
      // With one scale per row the chain runs on over the whole (rotated)
      // loop from the zeroed tmp; with groups of 128 K or more a wave's two
      // chunks of a stage lie in one group and are folded together.
      const bool first = GM == 1 ? true : GM == 2 ? c == 0 : false;
      const bool last = GM == 1 ? true : GM == 2 ? c == 1 : (it == nstages - 1 && c == 1);
      const u32x4 wv =
          *reinterpret_cast<const u32x4*>(sd + S::B_OFF + rw * 128 + 16 * ((4 * kh + 2 * c + h) ^ ((rw >> 1) & 7)));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const bf16x8 bo = b_operand(wv[s4], base);
        const int p = 16 * kh + 8 * c + 4 * h + s4;
        const bf16x8 ao =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sd + S::A_OFF + c32 * 512 + 16 * (p ^ (c32 & 15))));
        tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bo, (first && s4 == 0) ? f32x16{} : tmp, 0, 0, 0);
      }
      if (last) {  // last chunk of the group (or of the wave's part of it in this stage): fold with its scale
        const float sc = ROWSC ? rsc : *reinterpret_cast<const float*>(sd + S::SC_OFF + rw * 16 + (g & 3) * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __builtin_fmaf(sc, tmp[i], acc[i]);
      }
    }
    // Offset correction of the groups that end in this wave's chunks,
    // acc[m][n] += sc[n][g] * (-136 * sum of group g of A row m), as one fp32
    // MFMA 32x32x2 whose two K slots are the wave's two chunks (lane half h
    // holds chunk h: its group's correction if the group ends there, else 0,
    // and that group's scale).
    const int ch = st * 4 + 2 * kh + h;
    const int gh = ch >> a.gs_sh;
    const bool endh = GM == 0 ? (it == nstages - 1 && kh == 1 && h == 1) : (ch & (a.gs_ch - 1)) == a.gs_ch - 1;
    const bool any = GM == 0 ? (it == nstages - 1 && kh == 1) : GM == 1 ? true : ((st * 4 + 2 * kh + 1) & (a.gs_ch - 1)) == a.gs_ch - 1;
    if (any) {
      const float av =
          !endh ? 0.f : ROWSC ? corr0[c32] : -136.f * *reinterpret_cast<const float*>(sd + S::CR_OFF + c32 * 16 + (gh & 3) * 4);
      const float bv = ROWSC ? rsc : *reinterpret_cast<const float*>(sd + S::SC_OFF + rw * 16 + (gh & 3) * 4);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    // The next DMA goes out after this stage's compute: when the memory
    // pipeline's queues are full an issuing wave stalls in order, and issued
    // before the compute that stall would hold the MFMA and VALU work too.
    // The slot it fills was released at this iteration's barrier.
    if (it + kStages - 1 < nstages) {
      const int j = it + kStages - 1;
      issue_stage<S>(lds, rotated(j, rot, nstages), j % kStages, wave, lane, a.gs_sh, src);
    }
  }

  // epilogue; C layout: element 4i + j of a lane is row 8i + 4h + j, column lane & 31
  __syncthreads();  // every wave is done with the ring (no DMA outstanding after the last stage)
  float* xch = reinterpret_cast<float*>(lds);
  // the second K halves join the first
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) xch[(wl * 16 + i) * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += xch[(wl * 16 + i) * 64 + lane];
  }
  if constexpr (NM == 2) {
    // the up tiles join the gate tiles of the same columns
    __syncthreads();
    if (kh == 0 && wl >= HW / 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[((wl - HW / 2) * 16 + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (kh == 0 && wl < HW / 2) {
      const int col = n0 + wl * 32 + c32;
      const int pc = (col & ~7) | ((col & 7) < 4 ? 2 * (col & 7) : 2 * (col & 7) - 7);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * h + (i & 3);
        const float up = xch[(wl * 16 + i) * 64 + lane];
        const uint32_t hb = f32_to_bf16_bits(silu(acc[i]) * up);
        const float sum = group_sum<32>(bf16_bits_to_f32(hb));
        if (row < tl.mrows) {
          const int64_t pos = tl.pos0 + row;
          a.h[pos * a.N + pc] = (uint16_t)hb;
          if (c32 == 0) a.h32[pos * (a.N / 32) + col / 32] = sum;
        }
      }
    }
  } else {
    if (kh == 0) {
      const int col = n0 + wl * 32 + c32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * h + (i & 3);
        if (row < tl.mrows) a.out[(int64_t)s_pair[row] * a.N + col] = acc[i];
      }
    }
  }
}

template <int NM>
hipError_t launch_gemm(const GemmArgs<NM>& g, int blocks, hipStream_t st) {
  constexpr size_t lds_row = GemmShape<NM, true>::LDS, lds_grp = GemmShape<NM, false>::LDS;
  if (g.G == 1)
    hipLaunchKernelGGL((prefill_gemm_kernel<NM, 0>), dim3(blocks), dim3(kGT), lds_row, st, g);
  else if (g.gs_ch == 1)
    hipLaunchKernelGGL((prefill_gemm_kernel<NM, 1>), dim3(blocks), dim3(kGT), lds_grp, st, g);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<NM, 2>), dim3(blocks), dim3(kGT), lds_grp, st, g);
  return hipGetLastError();
}

// ---- 3. group sums of h ---------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void prefill_hsum_kernel(const float* __restrict__ h32, float* __restrict__ hsg,
                                                               const int* __restrict__ off, int E, int nblk, int G,
                                                               int nb32) {
  const int P = off[E];  // valid pairs
  const int64_t n = (int64_t)P * G;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t pos = i / G;
    const int g = (int)(i - pos * G);
    const float* src = h32 + pos * nblk + (int64_t)g * nb32;
    float s = 0.f;
    for (int j = 0; j < nb32; ++j) s += src[j];
    hsg[i] = s;
  }
}

// ---- 5. weighted combine in slot order ----------------------------------------------

__global__ __launch_bounds__(kThreads) void prefill_combine_kernel(const float* __restrict__ out,
                                                                  const int32_t* __restrict__ ids,
                                                                  const float* __restrict__ w, float* __restrict__ y,
                                                                  int T, int topk, int E, int H) {
  const int h4 = H / 4;
  const int64_t n = (int64_t)T * h4;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / h4;
    const int c = (int)(i - t * h4) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
      const int id = ids[t * topk + j];
      if (id < 0 || id >= E) continue;
      const float wt = w[t * topk + j];
      const f32x4 v = *reinterpret_cast<const f32x4*>(out + (t * topk + j) * H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(wt, v[q], acc[q]);
    }
    *reinterpret_cast<f32x4*>(y + t * H + c) = acc;
  }
}

// ---- workspace layout ---------------------------------------------------------------------

size_t al(size_t v) { return (v + 255) / 256 * 256; }

struct Layout {
  size_t hdr, off, tiles, sorted, xp, xsg, hs, h32, hsg, out, total;
  int mt_max;
};

Layout layout(int T, int topk, int E, int H, int I, int G_h, int G_i) {
  Layout L{};
  const size_t P = (size_t)T * topk;
  L.mt_max = (int)((P + kBM - 1) / kBM + (P < (size_t)E ? P : (size_t)E));
  size_t o = 0;
  L.hdr = o;    o += al(16);
  L.off = o;    o += al((size_t)(E + 1) * 4);
  L.tiles = o;  o += al((size_t)L.mt_max * sizeof(Tile));
  L.sorted = o; o += al(P * 4);
  L.xp = o;     o += al((size_t)T * H * 2);
  L.xsg = o;    o += al((size_t)T * G_h * 4);
  L.hs = o;     o += al(P * I * 2);
  L.h32 = o;    o += al(P * (I / 32) * 4);
  L.hsg = o;    o += al(P * G_i * 4);
  L.out = o;    o += al(P * H * 4);
  L.total = o;
  return L;
}

}  // namespace

bool moe_prefill_supported(int fmt, int topk, const ExpertArgs& e) {
  if (fmt != kFmtInt4 || topk < 1 || topk > kTopkMax) return false;
  if (e.E > kEMax || e.H % 512 || e.I % 256) return false;  // K in stages of 256; N-tiles 256 (down), 128 (gate+up)
  const int gsh = e.H / e.G_h, gsi = e.I / e.G_i;  // group sizes (== K when per row)
  if (gsh % 64 || gsi % 64) return false;
  // grouped scales move as aligned 16-byte pieces: G a multiple of 4, 16-byte aligned scale arrays
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (e.G_h > 1 && (e.G_h % 4 || !al16(e.gs) || !al16(e.us))) return false;
  if (e.G_i > 1 && (e.G_i % 4 || !al16(e.ds))) return false;
  if ((e.H / 32) > (1 << 16)) return false;
  return true;
}

size_t moe_prefill_workspace(int T, int topk, const ExpertArgs& e) {
  return layout(T, topk, e.E, e.H, e.I, e.G_h, e.G_i).total;
}

hipError_t launch_moe_prefill(int fmt, int xdt, const ExpertArgs& e, const void* x, const int32_t* ids,
                              const float* w, int T, int topk, float* y, void* ws, hipStream_t st) {
  if (!moe_prefill_supported(fmt, topk, e)) return hipErrorNotSupported;
  const Layout Ly = layout(T, topk, e.E, e.H, e.I, e.G_h, e.G_i);
  char* base = static_cast<char*>(ws);
  int* hdr = reinterpret_cast<int*>(base + Ly.hdr);
  int* off = reinterpret_cast<int*>(base + Ly.off);
  Tile* tiles = reinterpret_cast<Tile*>(base + Ly.tiles);
  int* sorted = reinterpret_cast<int*>(base + Ly.sorted);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base + Ly.xp);
  float* xsg = reinterpret_cast<float*>(base + Ly.xsg);
  uint16_t* hs = reinterpret_cast<uint16_t*>(base + Ly.hs);
  float* h32 = reinterpret_cast<float*>(base + Ly.h32);
  float* hsg = reinterpret_cast<float*>(base + Ly.hsg);
  float* out = reinterpret_cast<float*>(base + Ly.out);
  const int P = T * topk;

  // 1. prep
  PrepArgs pa{};
  pa.x = x;
  pa.ids = ids;
  pa.T = T;
  pa.topk = topk;
  pa.E = e.E;
  pa.H = e.H;
  pa.G = e.G_h;
  pa.nb32 = e.H / e.G_h / 32;
  pa.hdr = hdr;
  pa.off = off;
  pa.tiles = tiles;
  pa.sorted = sorted;
  pa.xp = xp;
  pa.xsg = xsg;
  const size_t lds_bucket = (size_t)(e.E + 2 * kThreads) * 4;
  const size_t lds_perm = (size_t)(e.H / 32) * 4;
  const size_t lds_prep = lds_bucket > lds_perm ? lds_bucket : lds_perm;
  if (xdt == kBF16)
    hipLaunchKernelGGL(prefill_prep_kernel<kBF16>, dim3(1 + T), dim3(kThreads), lds_prep, st, pa);
  else
    hipLaunchKernelGGL(prefill_prep_kernel<kF32>, dim3(1 + T), dim3(kThreads), lds_prep, st, pa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 2. gate + up
  {
    using Sh = GemmShape<2, false>;
    static_assert(Sh::BM == kBM, "tile rows");
    GemmArgs<2> g{};
    g.wq[0] = e.gq;
    g.wq[1] = e.uq;
    g.wsc[0] = e.gs;
    g.wsc[1] = e.us;
    g.rb = e.rb_h;
    g.eq = (int64_t)e.I * e.rb_h;
    g.es = (int64_t)e.I * e.G_h;
    g.N = e.I;
    g.K = e.H;
    g.G = e.G_h;
    g.gs_ch = e.H / e.G_h / 64;
    g.gs_sh = e.G_h == 1 ? 30 : __builtin_ctz(g.gs_ch);
    g.hdr = hdr;
    g.tiles = tiles;
    g.sorted = sorted;
    g.a = xp;
    g.asum = xsg;
    g.topk = topk;
    g.mt_max = Ly.mt_max;
    g.nt = e.I / Sh::BN;
    g.h = hs;
    g.h32 = h32;
    const int blocks = (Ly.mt_max * g.nt + 7) / 8 * 8;
    err = launch_gemm<2>(g, blocks, st);
    if (err != hipSuccess) return err;
  }

  // 3. group sums of h along I
  {
    const int nblk = e.I / 32;
    const int64_t n = (int64_t)P * e.G_i;
    int blocks = (int)((n + kThreads - 1) / kThreads);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(prefill_hsum_kernel, dim3(blocks), dim3(kThreads), 0, st, h32, hsg, off, e.E, nblk, e.G_i,
                       e.I / e.G_i / 32);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  // 4. down
  {
    using Sh = GemmShape<1, false>;
    static_assert(Sh::BM == kBM, "tile rows");
    GemmArgs<1> g{};
    g.wq[0] = e.dq;
    g.wsc[0] = e.ds;
    g.rb = e.rb_i;
    g.eq = (int64_t)e.H * e.rb_i;
    g.es = (int64_t)e.H * e.G_i;
    g.N = e.H;
    g.K = e.I;
    g.G = e.G_i;
    g.gs_ch = e.I / e.G_i / 64;
    g.gs_sh = e.G_i == 1 ? 30 : __builtin_ctz(g.gs_ch);
    g.hdr = hdr;
    g.tiles = tiles;
    g.sorted = sorted;
    g.a = hs;
    g.asum = hsg;
    g.topk = topk;
    g.mt_max = Ly.mt_max;
    g.nt = e.H / Sh::BN;
    g.out = out;
    const int blocks = (Ly.mt_max * g.nt + 7) / 8 * 8;
    err = launch_gemm<1>(g, blocks, st);
    if (err != hipSuccess) return err;
  }

  // 5. combine
  {
    const int64_t n = (int64_t)T * (e.H / 4);
    int blocks = (int)((n + kThreads - 1) / kThreads);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3(blocks), dim3(kThreads), 0, st, out, ids, w, y, T, topk, e.E,
                       e.H);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace qm
