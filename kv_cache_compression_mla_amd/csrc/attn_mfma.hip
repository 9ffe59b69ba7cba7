// Latent-space MLA decode attention on gfx950 bf16 MFMA.
//
// Every query head attends directly against the shared latent cache: the
// absorbed query q(i) = [W_UK(i)^T q_C(i) ; q_R(i)] is dotted with whole
// 576-wide rows [c_u ; kR_u], and the softmax weights combine the latents
// c_u themselves ("Understanding MLA" (Dong), section 4: the key
// up-projection moves onto the query; aicassindra MLA explainer, "End-to-end
// flow": content and rotary dot products summed, softmax over all history).
//
// The rotary part of the query (q_R, which dominates the scores at the
// DeepSeek-V3 widths) arrives as two bf16 terms, q_R = hi + lo, so that its
// rounding does not reach the softmax; the score chain adds the low term
// with four more MFMAs on the tile's rotary operands.
//
// Work decomposition: one workgroup = one sequence x one context chunk x all
// H heads, four waves. The heads that share a latent row form two dense
// contractions per 32-row tile:
//   S^T[row][head] = K_tile[row][0:576] . Q^T[0:576][head]     (MFMA 32x32x16)
//   O^T[col][head] += V_tile^T[col][rows] . P[rows][head]      (MFMA 32x32x16)
// with V_tile = K_tile[:, 0:512]. The score side is split by heads: wave w
// keeps the query block of heads 32w..32w+31 (32 x 576 bf16) in VGPRs, and
// computes their scores and softmax weights. The value side is split by
// latent columns: wave w accumulates O^T for columns 128w..128w+127 of all
// H heads (128 x 128 fp32 in AGPRs). The weights cross between the two
// splits through a small LDS buffer (bf16, 64 B per head per tile). Split
// this way, each wave reads only its quarter of V with transposed reads, 4x
// fewer than a head split, which is what bounds the value phase.
//
// Memory path: each 32-row tile is copied HBM -> LDS once per workgroup by
// LDS-DMA (global_load_lds, 16 B per lane: one copy moves one 1 KiB row
// latent, or the 128 B rotary parts of 8 rows), so nothing is staged in
// registers. Row addresses are wave-uniform (scalar base + per-lane offset),
// so a paged cache costs one scalar table read per 8 rows. LDS holds four
// latent stages (rows at a 1040-byte stride), three rotary slots (a tile's
// rotary part is dead once its scores are done; 128 B per row, 16-byte
// chunks XOR-swizzled) and two weight buffers (head records of four 16-byte
// slots, XOR-swizzled). The score operand is read with ds_read_b128 (lanes
// walk rows); the value operand, whose reduction index is the row, is read
// transposed with ds_read_b64_tr_b16 from the same row-major copy. A value
// block of 32 columns covers four runs of 8 columns 32 apart, which makes
// the transposed reads of 32 lanes tile all 64 banks. All three read
// patterns are bank-conflict free and every address is one per-lane base
// plus a compile-time offset. The query block is loaded coalesced (whole
// cache lines per load) and put in MFMA operand order through LDS before the
// first tile lands.
//
// Software pipeline (one wave per SIMD): iteration t runs the score MFMAs of
// tile t+1 with this wave's nine LDS-DMA copies of tile t+3 slotted between
// them, then the value MFMAs of tile t with the softmax of tile t+1 slotted
// between those (its weights go to the other weight buffer). One barrier per
// tile publishes the copies of tile t+1 and the weights of tile t, and frees
// the stages of tile t-1 for tile t+3.
//
// Softmax is online in base 2 (scale*log2(e) folded in) against a fixed
// per-head reference: the first tile's maximum. Weights exp2(x - m_ref) up to
// 2^32 are exact in fp32/bf16 range, and the final division by l removes the
// common factor, so no running rescale of O is needed and the accumulator is
// only ever touched by MFMA instructions (accumulate, and zero = 0*0 + 0),
// which keeps it resident in AGPRs. If a later tile's maximum exceeds a
// head's reference by more than 2^32 (adversarially growing scores), the
// workgroup redoes its chunk exactly: a scores-only pass finds every head's
// true maximum, and a second full pass uses it as the reference (weights
// <= 1). The result is the same softmax either way.
//
// Context chunks: every workgroup computes the same chunk plan from seq_lens
// (plan_chunks) and takes rows [r0, r1) of one sequence. A sequence cut into
// more than one chunk gets unnormalised (O, m, l) partials, merged exactly
// by combine_chunks. O goes out in fp16 with a power-of-two scale
// per (chunk, head): every element of the row is O * 2^-E with 2^E above the
// row's largest magnitude, so no element overflows and each keeps 11 bits
// relative to the row's maximum (half the bytes of float32 partials).
#include <type_traits>

#include <hip/hip_ext.h>

#include "mla_internal.hpp"

namespace mla {
#ifdef MLA_CLOCK_STAMPS
// Measurement build only (libmla_stamps.so; the library itself is built
// without it): every attention workgroup records the shader-clock counter
// (s_memtime, which counts shader cycles) and the 100 MHz real-time counter
// (s_memrealtime) at its start and at its end, so that clock_stamps.py can
// report cycles per workgroup and the clock each ran at. Wave 0 also records
// the shader clock at the boundaries of the kernel's phases (g_phase, eight
// per workgroup): start, plan done, first tile's scores and weights done,
// steady loop done, general loop done, last value step and fallback check
// done, (m, l) written, end.
constexpr int kStampSlots = 65536;
__device__ unsigned long long g_clock_stamps[4 * kStampSlots];
__device__ unsigned long long g_phase[8 * kStampSlots];
#define MLA_PHASE(i) (phase_t[i] = __builtin_amdgcn_s_memtime())
#else
#define MLA_PHASE(i) ((void)0)
#endif
namespace {

constexpr int DC = 512;               // latent width
constexpr int DW = 576;               // row width (latent + rotary key)
constexpr int ROW_BYTES = 2 * DW;     // 1152
constexpr int TILE = 32;              // rows per stage
constexpr int NTHREADS = 256;
constexpr int DMA_PER_WAVE = 9;       // 8 latent rows + 1 rotary block per tile
constexpr int QK_STEPS = DW / 16;     // 36 score MFMAs per tile
// A query row is [q_lat (512) ; q_R (64) ; q_R's low term (64)]: the rotary
// part dominates the scores at these widths, so it comes as two bf16 terms
// (nearest value, nearest value of the remainder) and the score chain runs
// four more MFMAs that reuse the tile's rotary operands for the low term.
constexpr int QW = DW + 64;           // query row elements
constexpr int QK_ALL = QK_STEPS + 4;  // score MFMAs per tile with the low term
constexpr int QK_DIST = 4;            // score-operand reads in flight
constexpr int PV_DIST = 3;            // value operands (pairs of reads) in flight
// Fast pass: a head's reference maximum is its first tile's maximum. A later
// tile exceeding it by more than this (log2 units) sends the workgroup to the
// exact two-pass fallback; otherwise probabilities stay in (0, 2^32].
constexpr float REF_GAP = 32.0f;

// LDS layout (bytes)
constexpr int LROW = 1040;                        // latent row stride (1024 + 16)
constexpr int LAT_STAGE = TILE * LROW;            // 33280
constexpr int NSTAGE = 4;
constexpr int ROPE_SLOT = TILE * 128;             // 4096
constexpr int NROPE = 3;
constexpr int P_BUF = 128 * 64;                   // weights: 128 heads x 32 rows bf16
constexpr int ROPE_OFF = NSTAGE * LAT_STAGE;      // 133120
constexpr int P_OFF = ROPE_OFF + NROPE * ROPE_SLOT;   // 145408
constexpr int LM_OFF = P_OFF + 2 * P_BUF;         // 161792: per-head (m, l), 1 KiB
constexpr int FLAG_OFF = LM_OFF + 128 * 8;        // 162816
constexpr int SMEM_BYTES = FLAG_OFF + 16;         // 162832 (of 163840)

// Cache addressing modes (template argument).
constexpr int CONTIG = 0;        // [B][capacity][576]
constexpr int PAGED8 = 1;        // paged, block_size >= 8: 8-row groups share a block
constexpr int PAGED_SMALL = 2;   // paged, block_size < 8
constexpr int GATHER_CONTIG = 3; // listed rows (sparse attention) of a contiguous cache
constexpr int GATHER_PAGED = 4;  // listed rows of a paged cache
// modes whose 8-row groups are not one contiguous run: one pointer per row
__host__ __device__ constexpr bool per_row(int pm) { return pm == PAGED_SMALL || pm >= GATHER_CONTIG; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct Params {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ cache;
  const int32_t* __restrict__ table;
  long long seq_stride;   // contiguous: capacity * DW elements
  int bs_log2, max_blocks;
  const int32_t* __restrict__ seq_lens;
  int B, H;
  int grid;               // workgroups launched (>= chunks in the plan)
  int splits;             // > 0: chunks per sequence (at most); 0: balanced plan
  float sl2;              // softmax scale * log2(e)
  float* o_lat;
  float* lse;
  uint16_t* part_o;       // [grid][H][512] fp16 partials O * 2^-E, by chunk
  float* part_ml;         // [grid][H][4]: m, l, E (the partial's scale exponent), unused
  int2* plan_seq;         // [B]: (first chunk, chunks) of each sequence
  const int32_t* indices; // gather modes: [B][topk] listed rows (seq_lens = counts)
  int topk;
  int qpt;                // query tokens per cached sequence (causal prefill), 1 for decode
};

// ---- chunk plan ----
// The rows of every sequence are cut into chunks of whole 32-row tiles, one
// chunk per workgroup; a sequence with more than one chunk gets (m, l, O)
// partials, merged by combine_chunks. Every workgroup computes the same plan
// from seq_lens (wave 0, in registers and LDS scratch) and finds its own
// chunk in it.
//  * splits > 0: sequence b gets ceil(L_b / c_b) chunks of c_b rows, c_b =
//    the multiple of 32 at or above L_b / splits.
//  * splits = 0 (balanced): the smallest chunk size C (a multiple of 32, at
//    least MIN_CHUNK rows) for which the chunk count sum_b ceil(L_b / C) fits
//    the grid; then sequence b gets ceil(L_b / C) chunks of near-equal size.
//    Long and short sequences of a ragged batch thus finish together, and a
//    batch of equal lengths gets ceil(L / C) chunks each.
// A sequence of length 0 gets one empty chunk (output: zeros, lse -inf).
constexpr int MIN_CHUNK = 128;
struct ChunkPlan {
  int b, r0, r1;   // sequence and rows [r0, r1)
  int start, n;    // the sequence's chunks: [start, start + n)
  int total;       // chunks in the plan (workgroups past it have no work)
  int g;           // this workgroup's chunk (index of its partials)
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
// Cross-lane operations of one fully active wave in VALU instructions only
// (DPP lane permutations within rows of 16 lanes, the row-pair and
// half-wave swaps v_permlane16_swap / v_permlane32_swap), not through the
// LDS permute unit: each step costs a few cycles instead of an LDS round
// trip, which matters on the dependent chains of the chunk plan.
// wave_reduce: every lane gets op over all 64 lanes. Each step combines a
// lane with its partner in an order both partners share, so every lane
// ends with the same bits (float sums included).
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  auto bits = [](T v) { return __builtin_bit_cast(int, v); };
  auto val = [](int v) { return __builtin_bit_cast(T, v); };
  x = op(x, val(__builtin_amdgcn_update_dpp(bits(x), bits(x), 0xB1, 0xf, 0xf, false)));   // lane ^ 1
  x = op(x, val(__builtin_amdgcn_update_dpp(bits(x), bits(x), 0x4E, 0xf, 0xf, false)));   // lane ^ 2
  x = op(x, val(__builtin_amdgcn_update_dpp(bits(x), bits(x), 0x141, 0xf, 0xf, false)));  // other quad of 8
  x = op(x, val(__builtin_amdgcn_update_dpp(bits(x), bits(x), 0x140, 0xf, 0xf, false)));  // other half of 16
  auto r = __builtin_amdgcn_permlane16_swap(bits(x), bits(x), false, false);   // rows 0|1, 2|3
  x = op(val(static_cast<int>(r[0])), val(static_cast<int>(r[1])));
  r = __builtin_amdgcn_permlane32_swap(bits(x), bits(x), false, false);        // halves
  return op(val(static_cast<int>(r[0])), val(static_cast<int>(r[1])));
}
__device__ __forceinline__ int wave_sum(int v) { return wave_reduce(v, [](int a, int b) { return a + b; }); }
__device__ __forceinline__ int wave_max(int v) { return wave_reduce(v, [](int a, int b) { return max(a, b); }); }
__device__ __forceinline__ int wave_min(int v) { return wave_reduce(v, [](int a, int b) { return min(a, b); }); }
// sum of non-negative 64-bit values below 2^55 per lane: 24-bit low parts
// and the high parts summed separately (64 * 2^24 fits in 31 bits)
__device__ __forceinline__ long long wave_sum64(long long v) {
  const int lo = wave_sum(static_cast<int>(v & 0xffffff));
  const int hi = wave_sum(static_cast<int>(v >> 24));
  return (static_cast<long long>(hi) << 24) + lo;
}
// Inclusive prefix sum over the 64 lanes: within each row of 16 by shifted
// adds (a lane with no source lane adds 0), then the totals of the rows
// before it.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // lane - 1 within the row
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // lane - 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // lane - 4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // lane - 8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Chunks of one sequence of length L, given its target count t >= 1.
__device__ __forceinline__ void seq_chunks(int L, int t, int* rows, int* n) {
  const int c = max(TILE, ceil_div(ceil_div(L, t), TILE) * TILE);
  *rows = c;
  *n = max(1, ceil_div(L, c));
}

// Every thread of the workgroup calls this; the result is the same in all.
// scratch: LDS for B ints (free until the first tile copy); res: 8 ints of
// LDS that stay untouched until the epilogue.
__device__ ChunkPlan plan_chunks(const Params& p, int* scratch, int* res) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    for (int i = lane; i < p.B; i += 64) scratch[i] = virt_len(p.seq_lens, i, p.qpt);
    // (LDS writes and reads below are by this wave only, in order)
    long long sum = 0;
    int mx = 0, mn = 0x7fffffff;
    for (int i = lane; i < p.B; i += 64) {
      const int L = scratch[i];
      sum += L;
      mx = max(mx, L);
      mn = min(mn, L);
    }
    const int lmax = wave_max(mx), lmin = wave_min(mn);
    int target_rows = 0;   // balanced: the chunk size C
    if (p.splits == 0) {
      sum = wave_sum64(sum);
      const int avg = static_cast<int>((sum + p.grid - 1) / p.grid);
      // chunks for chunk size 32k: sum_b max(1, ceil(L_b / 32k)), which does
      // not grow with k
      auto chunks = [&](int k) {
        const int c = k * TILE;
        int cnt = 0;
        for (int i = lane; i < p.B; i += 64) cnt += max(1, ceil_div(scratch[i], c));
        return wave_sum(cnt);
      };
      // the smallest k with chunks(k) <= grid lies in [klo, khi]: no chunk
      // size below the average fits, and one chunk per sequence always does.
      // The lower end is tried first: it is the answer for equal lengths.
      int klo = ceil_div(max(MIN_CHUNK, avg), TILE);
      int khi = max(klo, ceil_div(max(lmax, 1), TILE));
      if (klo < khi) {
        if (chunks(klo) <= p.grid) khi = klo;
        else ++klo;
      }
      while (klo < khi) {
        const int mid = (klo + khi) >> 1;
        if (chunks(mid) <= p.grid) khi = mid;
        else klo = mid + 1;
      }
      target_rows = klo * TILE;
    }
    // chunk counts, then an exclusive scan over the sequences in lane-major
    // blocks: lane l owns sequences [l * per, (l + 1) * per)
    const int per = ceil_div(p.B, 64);
    int local = 0;
    for (int i = lane * per; i < min(p.B, (lane + 1) * per); ++i) {
      const int L = scratch[i];
      int rows, n;
      seq_chunks(L, p.splits > 0 ? p.splits : max(1, ceil_div(L, target_rows)), &rows, &n);
      local += n;
    }
    const int incl = wave_incl_scan(local, lane);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    int start = incl - local;
    // Workgroup -> chunk. When every sequence has the same length (so the
    // same chunk count n) and B is a multiple of 8, the n chunks of a
    // sequence take workgroups 8 apart in launch order (groups of 8
    // sequences x n chunks), which dispatch places on one XCD, so they read
    // the sequence's query block through that XCD's L2. Otherwise
    // workgroup x takes chunk x. Chunk indices stay in prefix order.
    int g = blockIdx.x;
    if (lmin == lmax && (p.B & 7) == 0) {
      int rows, n;
      seq_chunks(lmax, p.splits > 0 ? p.splits : max(1, ceil_div(lmax, target_rows)), &rows, &n);
      if (g < n * p.B) {
        const int grp = g / (8 * n), r = g % (8 * n);
        g = n * (8 * grp + (r & 7)) + (r >> 3);
      }
    }
    for (int i = lane * per; i < min(p.B, (lane + 1) * per); ++i) {
      const int L = scratch[i];
      int rows, n;
      seq_chunks(L, p.splits > 0 ? p.splits : max(1, ceil_div(L, target_rows)), &rows, &n);
      if (g >= start && g < start + n) {
        const int k = g - start;
        res[0] = i;
        res[1] = k * rows;
        res[2] = min((k + 1) * rows, L);
        res[3] = start;
        res[4] = n;
      }
      start += n;
    }
    if (lane == 0) {
      res[5] = total;
      res[6] = g;
      if (g >= total) res[0] = -1;
    }
  }
  __syncthreads();
  ChunkPlan c;
  c.b = __builtin_amdgcn_readfirstlane(res[0]);
  c.r0 = __builtin_amdgcn_readfirstlane(res[1]);
  c.r1 = __builtin_amdgcn_readfirstlane(res[2]);
  c.start = __builtin_amdgcn_readfirstlane(res[3]);
  c.n = __builtin_amdgcn_readfirstlane(res[4]);
  c.total = __builtin_amdgcn_readfirstlane(res[5]);
  c.g = __builtin_amdgcn_readfirstlane(res[6]);
  return c;
}

// XOR swizzle of the 16-byte chunks of a packed 128-byte rotary row: 16
// lanes reading one chunk of 16 rows hit distinct bank groups.
__device__ __forceinline__ int rope_sw(int r) { return (r >> 1) & 7; }

// First column of value block cb: blocks hold columns
// colbase + {0..7} + 32 * {0..3}. Blocks 4w..4w+3 cover columns
// 128w..128w+127.
__host__ __device__ constexpr int colbase(int cb) { return 8 * (cb % 4) + 128 * (cb / 4); }

// Byte offset of weight slot (t, h) of head `head` in a weight buffer: a
// head record is 64 B (logical rows 16t + 8h + 0..7 in slot 2t + h), slots
// XOR-swizzled by (head >> 2) & 3 so that 16 consecutive heads hit distinct
// bank groups.
__device__ __forceinline__ int p_slot(int head, int t, int h) {
  return head * 64 + 16 * ((2 * t + h) ^ ((head >> 2) & 3));
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8]; unconstrained fields at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Row u of sequence b. Called with wave-uniform arguments only; the block
// table is read through the constant address space so that the read is a
// scalar load (it must not wait on the vector-memory counter, which also
// tracks the LDS-DMA copies in flight).
typedef __attribute__((address_space(4))) const int32_t const_i32;
template <int PM>
__device__ __forceinline__ const uint16_t* row_ptr(const Params& p, int b, int u) {
  if constexpr (PM == GATHER_CONTIG || PM == GATHER_PAGED) {
    const const_i32* ix = (const const_i32*)(p.indices);   // listed position of entry u
    u = ix[static_cast<long long>(b) * p.topk + u];
  }
  if constexpr (PM == CONTIG || PM == GATHER_CONTIG) {
    return p.cache + b * p.seq_stride + static_cast<long long>(u) * DW;
  } else {
    const const_i32* tab = (const const_i32*)(p.table);
    const int blk = tab[b * p.max_blocks + (u >> p.bs_log2)];
    return p.cache + ((static_cast<long long>(blk) << p.bs_log2) + (u & ((1 << p.bs_log2) - 1))) * DW;
  }
}

// LDS-DMA copies, written as inline asm so that the compiler adds none of its
// own (conservative, vmcnt(0)) waits in front of later LDS reads; the kernel
// waits for them explicitly (wait_vmcnt + barrier). A copy has no register
// result and its address operands are read at issue. Every lane moves 16
// bytes to LDS at lds + 16 * lane.
//   copy_s: from row + voff (row wave-uniform, voff per lane)
//   copy_v: from a per-lane 64-bit address
__device__ __forceinline__ void copy_s(const uint16_t* row, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:0"
               :: "s"(lds), "v"(voff), "s"(row));
}
__device__ __forceinline__ void copy_v(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(gptr));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// This wave's share of one tile copy: the latents of tile rows 8w..8w+7 (one
// copy each) and the rotary parts of the same rows (one copy; lane -> row
// 8w + (lane >> 3), chunk (lane & 7) ^ rope_sw(row)). Rows at or past
// row_end are replaced by row_end - 1 (a real row, later masked out of the
// softmax), so no invalid address is ever read. In CONTIG and PAGED8 modes
// the rows of the group lie in one contiguous run (a group of 8 rows starting
// at a multiple of 8 never crosses a block of >= 8 rows), so every copy is a
// uniform base plus a per-lane offset.
struct TileCopy {
  const uint16_t* row[8];
  const uint16_t* rope_base;   // CONTIG / PAGED8
  uint32_t rope_voff;
  const uint16_t* rope_ptr;    // PAGED_SMALL: per lane
};

template <int PM>
__device__ __forceinline__ TileCopy plan_copy(const Params& p, int b, int r0, int row_end, int w, int lane) {
  TileCopy c;
  const int first = r0 + 8 * w;
  const int last = row_end - 1;
  const int j = lane >> 3;
  const int chunk = (lane & 7) ^ rope_sw(8 * w + j);
  if constexpr (per_row(PM)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c.row[k] = row_ptr<PM>(p, b, min(first + k, last));
    const uint16_t* mine = c.row[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mine = (j == k) ? c.row[k] : mine;
    c.rope_ptr = mine + DC + 8 * chunk;
    c.rope_base = nullptr;
    c.rope_voff = 0;
  } else {
    const int g0 = min(first, last);
    const uint16_t* base = row_ptr<PM>(p, b, g0);
#pragma unroll
    for (int k = 0; k < 8; ++k) c.row[k] = base + (min(first + k, last) - g0) * DW;
    c.rope_base = base;
    c.rope_voff = (min(first + j, last) - g0) * ROW_BYTES + 2 * DC + 16 * chunk;
    c.rope_ptr = nullptr;
  }
  return c;
}

// Copy k (0..8) of this wave's share: latents into the latent stage at LDS
// address lat, the rotary block into the rotary slot at LDS address rope.
template <int PM>
__device__ __forceinline__ void copy_part(const TileCopy& c, int k, uint32_t lat, uint32_t rope, int w,
                                          uint32_t lane_off) {
  if (k < 8) {
    copy_s(c.row[k], lane_off, lat + (8 * w + k) * LROW);
  } else if constexpr (per_row(PM)) {
    copy_v(c.rope_ptr, rope + w * 1024);
  } else {
    copy_s(c.rope_base, c.rope_voff, rope + w * 1024);
  }
}

// Copy k (0..8) of this wave's share of an interior tile (all 32 rows before
// row_end) in CONTIG or PAGED8 mode: the wave's 8-row group starts at `group`
// (one contiguous run of rows), latent row k at group + k rows goes to LDS
// lat + k * LROW, the rotary block (per-lane offset rope_voff from group) to
// rope. No clamping and no table read per copy: one 64-bit scalar add and
// the M0 update.
template <int K>
__device__ __forceinline__ void copy_interior(const uint16_t* group, uint32_t lane_off, uint32_t rope_voff,
                                              uint32_t lat, uint32_t rope) {
  if constexpr (K < 8) {
    asm volatile("s_add_i32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3 offset:0"
                 :: "s"(lat), "i"(K * LROW), "v"(lane_off), "s"(group + K * DW));
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:0"
                 :: "s"(rope), "v"(rope_voff), "s"(group));
  }
}
__device__ __forceinline__ void copy_interior_k(int k, const uint16_t* group, uint32_t lane_off,
                                                uint32_t rope_voff, uint32_t lat, uint32_t rope) {
  switch (k) {   // k is a constant after unrolling: one case survives
    case 0: copy_interior<0>(group, lane_off, rope_voff, lat, rope); break;
    case 1: copy_interior<1>(group, lane_off, rope_voff, lat, rope); break;
    case 2: copy_interior<2>(group, lane_off, rope_voff, lat, rope); break;
    case 3: copy_interior<3>(group, lane_off, rope_voff, lat, rope); break;
    case 4: copy_interior<4>(group, lane_off, rope_voff, lat, rope); break;
    case 5: copy_interior<5>(group, lane_off, rope_voff, lat, rope); break;
    case 6: copy_interior<6>(group, lane_off, rope_voff, lat, rope); break;
    case 7: copy_interior<7>(group, lane_off, rope_voff, lat, rope); break;
    default: copy_interior<8>(group, lane_off, rope_voff, lat, rope); break;
  }
}

// Workgroup barrier; this wave's LDS writes (the softmax weights) complete
// first, so that every wave reads them after the barrier.
__device__ __forceinline__ void block_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Keeps a value in a register at this point of the instruction stream: the
// computation producing it cannot sink below, nor its users rise above, the
// neighbouring MFMA statements. Used to slot VALU work between MFMAs.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }
template <typename T>
__device__ __forceinline__ T pinned(T x) { asm volatile("" : "+v"(x)); return x; }

// MFMA instructions issued from inline asm are invisible to the compiler's
// hazard tracking. Where an operand is produced by the VALU (the zero
// operand) the asm carries the VALU-write to MFMA-read wait states itself;
// where the VALU reads an MFMA result (the scores), explicit nops follow the
// last MFMA of the chain. All other operands come from LDS reads, whose
// completion the compiler's counter waits cover; a CPU test scans the
// compiled ISA for every VALU write close before an MFMA that reads it.
#define MLA_MFMA_PRE "s_nop 4\n\t"

// acc = 0 * 0 + 0: clears an accumulator block through the MFMA unit.
__device__ __forceinline__ void mfma_zero(f32x16& acc, const bf16x8& zero8) {
  asm volatile(MLA_MFMA_PRE "v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero8));
}

// Plain VALU maxima (inline asm: the inputs are finite or -inf, so none of
// the NaN canonicalisation the compiler adds around fmaxf is needed).
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The fp16 value in the low 16 bits of u, as a float (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
}

// max / sum over both half-waves (lanes l and l ^ 32), VALU only
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// NW = H / 32 head blocks. Waves w >= NW (H < 128) compute the scores of head
// block w % NW a second time and write identical weights, which keeps every
// wave on one branch-free path.
template <int NW, int PM>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(Params p) {
  __shared__ __align__(1024) char smem[SMEM_BYTES];
  const uint32_t smem_lds = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int hq = w % NW;              // this wave's score head block
  const int qhead = 32 * hq + l32;    // this lane's score head

#ifdef MLA_CLOCK_STAMPS
  const unsigned long long stamp_t0 = __builtin_amdgcn_s_memtime(), stamp_r0 = __builtin_amdgcn_s_memrealtime();
#endif
  const ChunkPlan plan = plan_chunks(p, reinterpret_cast<int*>(smem), reinterpret_cast<int*>(smem + LM_OFF));
#ifdef MLA_CLOCK_STAMPS
  unsigned long long phase_t[8] = {stamp_t0, 0, 0, 0, 0, 0, 0, 0};
  MLA_PHASE(1);
#endif
  if (plan.b < 0) return;             // no chunk for this workgroup
  const int b = plan.b;
  const int bc = p.qpt == 1 ? b : b / p.qpt;   // the cached sequence it reads
  const int gi = plan.g;              // chunk index (partials)
  const bool single = plan.n == 1;    // whole sequence here: final output
  if (tid == 0 && plan.r0 == 0) p.plan_seq[b] = int2{plan.start, plan.n};
  const int row_begin = plan.r0;
  const int row_end = plan.r1;

  if (row_begin >= row_end) {
    // Empty sequence (its single chunk): zeros, lse -inf.
    if (w < NW) {
      float* o = p.o_lat + (static_cast<long long>(b) * p.H + qhead) * DC;
      for (int c = h * 256; c < h * 256 + 256; c += 4)
        *reinterpret_cast<f32x4*>(o + c) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p.lse && h == 0) p.lse[b * p.H + qhead] = -INFINITY;
    }
    return;
  }
  const int ntiles = (row_end - row_begin + TILE - 1) / TILE;
  const uint32_t lane_off = 16 * lane;

  // Query of this lane's head in MFMA B-operand order: step s, half h holds
  // columns 16s + 8h .. 16s + 8h + 7. A query row is 1280 bytes, five
  // segments of 256. Loaded coalesced first: load i of a wave brings segment
  // i / 8 of the four heads 4 (i % 8) .. 4 (i % 8) + 3 of its block, 16 lanes
  // per head and 16 bytes per lane, lane position p holding piece
  // (p - head) mod 16 of the segment (eight whole cache lines per load, where
  // one lane per head would touch 32 lines per load, each four times). The
  // operand order is then made through LDS (qperm, after the first copies are
  // issued): steps 8r .. 8r + 7 use exactly loads 8r .. 8r + 7.
  bf16x8 qreg[QK_ALL];
  {
    const uint16_t* qb = p.q + (static_cast<long long>(b) * p.H + 32 * hq) * QW;
    const int pos = lane & 15;
#pragma unroll
    for (int i = 0; i < QK_ALL; ++i) {
      const int hd = 4 * (i % 8) + (lane >> 4);
      qreg[i] = *reinterpret_cast<const bf16x8*>(qb + hd * QW + 128 * (i / 8) + 8 * ((pos - hd) & 15));
    }
  }
  // Operand order through this wave's 8 KiB of LDS in the fourth tile stage
  // (untouched until tile 3's copy, after the first barrier of the loop), five
  // rounds: the round's eight loads are written as they came (1 KiB each,
  // contiguous), then step s = 8r + j of head l32 is read from load 8r + l32 / 4,
  // head slot l32 % 4, position (2j + h + l32) mod 16, which for the 16 heads
  // of a read pass are 16 distinct bank groups. Wave-local: LDS operations of
  // a wave complete in order.
  static_assert(QK_ALL == 5 * 8 && 2 * QW == 5 * 256, "five rounds of eight loads, five 256-byte segments");
  static_assert(4 * 8192 <= LAT_STAGE, "the four waves' query staging fits one tile stage");
  auto qperm = [&]() {
    char* qs = smem + 3 * LAT_STAGE + 8192 * w;
#pragma unroll
    for (int r = 0; r < QK_ALL / 8; ++r) {
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<bf16x8*>(qs + 1024 * j + 16 * lane) = qreg[8 * r + j];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qreg[8 * r + j] = *reinterpret_cast<const bf16x8*>(qs + 1024 * (l32 >> 2) + 256 * (l32 & 3) +
                                                           16 * ((2 * j + h + l32) & 15));
    }
  };

  // O^T accumulators: block NW*c + hb holds columns of value block 4w + c
  // against heads 32hb..32hb+31.
  const bf16x8 zero8 = {};
  f32x16 oacc[4 * NW];
#pragma unroll
  for (int i = 0; i < 4 * NW; ++i) mfma_zero(oacc[i], zero8);
  float m_ref = -INFINITY;   // reference maximum, log2 units (score heads)
  float l_run = 0.f;         // this lane's partial weight sum

  // Per-lane LDS bases; every other part of an operand address is a
  // compile-time immediate of the unrolled loops below.
  //  score operand: row l32, latent chunk 2s + h at 16 * (2s + h)
  const int qk_base = l32 * LROW + 16 * h;
  //  rotary part of row l32: chunk c' at 16 * (c' ^ rope_sw(l32))
  const int rp_base = l32 * 128;
  const int rp_sw = rope_sw(l32);
  //  value operand, transposed read: in its 16-lane group a lane supplies row
  //  16t + 8k + 4*(g16>>1) + tr_e, 8 bytes at column colbase(cb) + 32*tr_q + 4*(g16&1)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_base = (4 * (g16 >> 1) + (i16 >> 2)) * LROW + 64 * (i16 & 3) + 8 * (g16 & 1) + 2 * colbase(4 * w);
  //  weight operand of head 32hb + l32, slot (t, h): p_slot minus 2048 hb
  const int pr_base0 = p_slot(l32, 0, h), pr_base1 = p_slot(l32, 1, h);

  auto lat_off = [&](int t) { return (t % NSTAGE) * LAT_STAGE; };
  auto rope_off = [&](int t) { return ROPE_OFF + (t % NROPE) * ROPE_SLOT; };
  auto p_off = [&](int t) { return P_OFF + (t & 1) * P_BUF; };
  auto tile_r0 = [&](int t) { return row_begin + t * TILE; };
  auto tile_nv = [&](int t) { return min(TILE, row_end - tile_r0(t)); };
  auto copy_tile = [&](int t) {
    const TileCopy c = plan_copy<PM>(p, bc, tile_r0(t), row_end, w, lane);
#pragma unroll
    for (int k = 0; k < DMA_PER_WAVE; ++k)
      copy_part<PM>(c, k, smem_lds + lat_off(t), smem_lds + rope_off(t), w, lane_off);
  };

  // S^T[row][head] of one tile over all 576 columns, one accumulation chain;
  // between(s) runs after the MFMA of step s.
  auto qk = [&](int t, f32x16& acc, auto&& between) {
    const char* lat = smem + lat_off(t);
    const char* rope = smem + rope_off(t);
    auto operand = [&](int s) -> bf16x8 {
      const char* ap = (s < 32) ? lat + qk_base + 32 * s
                                : rope + rp_base + 16 * ((2 * (s - 32) + h) ^ rp_sw);
      return *reinterpret_cast<const bf16x8*>(ap);
    };
    bf16x8 a[QK_DIST];
#pragma unroll
    for (int i = 0; i < QK_DIST; ++i) a[i] = operand(i);
#pragma unroll
    for (int s = 0; s < QK_ALL; ++s) {
      const bf16x8 cur = a[s % QK_DIST];
      // steps 36..39 (the rotary low term) reuse the rotary operands of steps
      // 32..35, which stay in the ring: no refill past the last real step
      if (s + QK_DIST < QK_STEPS) a[s % QK_DIST] = operand(s + QK_DIST);
      if (s == 0)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(cur), "v"(qreg[s]));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(cur), "v"(qreg[s]));
      between(s);
    }
    // the VALU reads the scores next
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
  };

  // O^T[cols of this wave][all heads] += V^T P for tile t, weights from the
  // weight buffer of tile t. Steps run (k-step, c, hb) in that order;
  // between(step) runs after each MFMA.
  constexpr int PV_STEPS = 8 * NW;
  auto pv = [&](int t, auto&& between) {
    const char* lat = smem + lat_off(t);
    const char* pw = smem + p_off(t);
    auto v_operand = [&](int vi) -> bf16x8 {   // vi = 4 * kstep + c
      const char* a = lat + tr_base + (16 * LROW) * (vi >> 2) + 16 * (vi & 3);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * LROW));
      return __builtin_bit_cast(bf16x8, (s16x8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    auto p_operand = [&](int hb, int ks) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(pw + (ks ? pr_base1 : pr_base0) + 2048 * hb);
    };
    bf16x8 P[NW];
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) P[hb] = p_operand(hb, 0);
    bf16x8 V[PV_DIST];
#pragma unroll
    for (int i = 0; i < PV_DIST; ++i) V[i] = v_operand(i);
    int step = 0;
#pragma unroll
    for (int vi = 0; vi < 8; ++vi) {
      const bf16x8 cur = V[vi % PV_DIST];
      if (vi + PV_DIST < 8) V[vi % PV_DIST] = v_operand(vi + PV_DIST);
      const int c = vi & 3;
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(oacc[NW * c + hb]) : "v"(cur), "v"(P[hb]));
        if (vi == 3) P[hb] = p_operand(hb, 1);   // last use of the first k-step's weights
        between(step++);
      }
    }
  };

  // ---- softmax of one tile, as a sequence of small steps ----
  // x: the tile's raw scores (lane: head qhead, register r <-> row
  // 8*(r>>2) + 4h + (r&3)); nv: valid rows; set_ref: this tile sets the
  // reference (fast pass, first tile). Writes the tile's bf16 weights to its
  // weight buffer (slot (t, h) holds registers 8t..8t+7) and adds them into
  // l_run. In log2 units a score is x = s * sl2; the tile maximum is taken on
  // raw scores (scaling by sl2 > 0 preserves order), m = round(max * sl2),
  // and each weight is exp2(fma(s, sl2, -m_ref)). The normaliser sums the
  // bf16-rounded weights, i.e. exactly the weights the value MFMAs apply (so
  // a single row reproduces its latent exactly). Each step is a few
  // independent VALU instructions, sized to sit under one MFMA.
  struct Soft {
    f32x16 x;
    float mx[7];
    float psum;
    bf16x8 pb[2];
  };
  constexpr int SM_STEPS = 29;
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  // Every step pins the values it reads on entry and those it writes on
  // exit (pin/pinned: empty volatile asm), so its instructions can move
  // neither above nor below the MFMAs around it.
  auto soft_step = [&](Soft& S, int k, int nv, bool set_ref, bool& grew, int pbuf) {
    if (k == 0) {
#pragma unroll
      for (int r = 0; r < 12; ++r) S.x[r] = pinned(S.x[r]);
      if (nv < TILE) {                  // mask rows past the end (last tile only)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * h + (r & 3) >= nv) S.x[r] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) S.mx[i] = pinned(max3(S.x[3 * i], S.x[3 * i + 1], S.x[3 * i + 2]));
    } else if (k == 1) {
#pragma unroll
      for (int r = 12; r < 16; ++r) S.x[r] = pinned(S.x[r]);
      S.mx[4] = max3(S.x[12], S.x[13], S.x[14]);
      S.mx[5] = pinned(max3(S.mx[0], S.mx[1], S.x[15]));
      S.mx[6] = pinned(max3(S.mx[2], S.mx[3], S.mx[4]));
    } else if (k == 2) {
      S.mx[0] = pinned(max_halves(max2(S.mx[5], S.mx[6])));
    } else if (k == 3) {
      const float tmax = S.mx[0] * p.sl2;
      if (set_ref) m_ref = tmax;
      else grew = grew || (tmax > m_ref + REF_GAP);
      pin(m_ref);
      S.psum = 0.f;
    } else if (k < 20) {                // 4..19: one weight per step
      const int r = k - 4;
      S.x[r] = pinned(__builtin_amdgcn_exp2f(__builtin_fmaf(pinned(S.x[r]), p.sl2, -m_ref)));
    } else if (k < 28) {                // 20..27: pack a pair to bf16, add it to the sum
      const int i = k - 20, t = i >> 2, e = i & 3;
      const float x0 = pinned(S.x[8 * t + 2 * e]), x1 = pinned(S.x[8 * t + 2 * e + 1]);
      const bf16x2 v2 = __builtin_convertvector((f32x2{x0, x1}), bf16x2);
      S.pb[t][2 * e] = v2[0];
      S.pb[t][2 * e + 1] = v2[1];
      S.psum = pinned(__builtin_amdgcn_fdot2_f32_bf16(v2, ones2, S.psum, false));
      if (e == 3) {
        pin(S.pb[t]);
        char* dst = smem + pbuf + 2048 * hq + (t ? pr_base1 : pr_base0);
        *reinterpret_cast<bf16x8*>(dst) = S.pb[t];
      }
    } else {
      l_run += S.psum;
    }
  };

  // ---- fast pass (reference from the first tile) or, with fixed_ref, the
  // exact second pass against known maxima ----
  auto full_pass = [&](bool fixed_ref) -> bool {
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
      if (j < ntiles) copy_tile(j);
    if (!fixed_ref) {
      // the query loads (issued first) are done; the tile copies may fly
      if (ntiles >= 3) wait_vmcnt<3 * DMA_PER_WAVE>();
      else if (ntiles == 2) wait_vmcnt<2 * DMA_PER_WAVE>();
      else wait_vmcnt<DMA_PER_WAVE>();
      qperm();
    }
    // Wait for tile 0; tiles 1 and 2 may still fly. The loop's waits count
    // only these copies: nothing else in flight.
    if (ntiles >= 3) wait_vmcnt<2 * DMA_PER_WAVE>();
    else if (ntiles == 2) wait_vmcnt<DMA_PER_WAVE>();
    else wait_vmcnt<0>();
    block_barrier();
    bool grew = false;
    {
      Soft S;
      qk(0, S.x, [](int) {});
#pragma unroll
      for (int k = 0; k < SM_STEPS; ++k) soft_step(S, k, tile_nv(0), !fixed_ref, grew, p_off(0));
    }
    if (!fixed_ref) MLA_PHASE(2);
    // Iteration t: tile t+1 has landed (only the copies of tile t+2 may
    // still fly), every wave has written the weights of tile t and is past
    // tile t-1, whose stages tile t+3 reuses.
    int t = 0;
    if constexpr (!per_row(PM)) {
      // Steady state (t + 4 < ntiles): tiles t+1 and t+3 are interior (32
      // rows before row_end), so no row is masked and the copies of tile t+3
      // need no clamping; the general loop below takes the last iterations.
      const int jr = lane >> 3;
      const uint32_t rope_voff = jr * ROW_BYTES + 2 * DC + 16 * ((lane & 7) ^ rope_sw(8 * w + jr));
      for (; t + 4 < ntiles; ++t) {
        wait_vmcnt<DMA_PER_WAVE>();
        block_barrier();
        const uint16_t* group = row_ptr<PM>(p, bc, tile_r0(t + 3) + 8 * w);
        const uint32_t lat3 = smem_lds + lat_off(t + 3) + 8 * w * LROW;
        const uint32_t rope3 = smem_lds + rope_off(t + 3) + w * 1024;
        Soft N;
        qk(t + 1, N.x, [&](int s) {
          if (s % 4 == 1 && s / 4 < DMA_PER_WAVE) copy_interior_k(s / 4, group, lane_off, rope_voff, lat3, rope3);
        });
        const int pb_next = p_off(t + 1);
        pv(t, [&](int step) {
          if (step < SM_STEPS) soft_step(N, step, TILE, false, grew, pb_next);
        });
#pragma unroll
        for (int k = PV_STEPS; k < SM_STEPS; ++k) soft_step(N, k, TILE, false, grew, pb_next);
      }
    }
    if (!fixed_ref) MLA_PHASE(3);
    for (; t + 1 < ntiles; ++t) {
      if (t + 2 < ntiles) wait_vmcnt<DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      block_barrier();
      const bool copy_next = t + 3 < ntiles;
      const TileCopy c = plan_copy<PM>(p, bc, tile_r0(copy_next ? t + 3 : t), row_end, w, lane);
      const uint32_t lat3 = smem_lds + lat_off(t + 3), rope3 = smem_lds + rope_off(t + 3);
      Soft N;
      qk(t + 1, N.x, [&](int s) {
        if (s % 4 == 1 && s / 4 < DMA_PER_WAVE && copy_next) copy_part<PM>(c, s / 4, lat3, rope3, w, lane_off);
      });
      const int nv = tile_nv(t + 1), pb_next = p_off(t + 1);
      pv(t, [&](int step) {
        if (step < SM_STEPS) soft_step(N, step, nv, false, grew, pb_next);
      });
#pragma unroll
      for (int k = PV_STEPS; k < SM_STEPS; ++k) soft_step(N, k, nv, false, grew, pb_next);
    }
    // last tile: its weights are complete once every wave is here
    if (!fixed_ref) MLA_PHASE(4);
    block_barrier();
    pv(t, [](int) {});
    return grew;
  };

  // ---- fallback scores-only pass: exact per-head maximum over the chunk ----
  // Copies run two tiles ahead (iteration t refills the stages of tile t-2
  // and the rotary slot of tile t-1, both finished before its barrier).
  auto max_pass = [&]() -> float {
    float m_seen = -INFINITY;
    copy_tile(0);
    if (1 < ntiles) copy_tile(1);
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) wait_vmcnt<DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      block_barrier();
      if (t + 2 < ntiles) copy_tile(t + 2);
      f32x16 x;
      qk(t, x, [](int) {});
      const int nv = tile_nv(t);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * h + (r & 3) >= nv) x[r] = -INFINITY;
      float tmax = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = max2(tmax, x[r]);
      m_seen = max2(m_seen, max_halves(tmax) * p.sl2);
    }
    return m_seen;
  };

  int* wg_flag = reinterpret_cast<int*>(smem + FLAG_OFF);
  bool grew = full_pass(false);
  // did any head in the workgroup outgrow its reference?
  if (tid == 0) *wg_flag = 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(grew) != 0 && lane == 0) *wg_flag = 1;
  __syncthreads();
  MLA_PHASE(5);
  if (*wg_flag != 0) {
    __syncthreads();
    const float m_exact = max_pass();
    __syncthreads();
    m_ref = m_exact;
    l_run = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * NW; ++i) mfma_zero(oacc[i], zero8);
    full_pass(true);
  }

  // Per-head (m, l) through LDS: the value split needs every head's l.
  float* lm = reinterpret_cast<float*>(smem + LM_OFF);
  const float l_tot = sum_halves(l_run);
  if (w < NW && h == 0) {
    lm[2 * qhead] = m_ref;
    lm[2 * qhead + 1] = l_tot;
    if (single) {
      if (p.lse) p.lse[b * p.H + qhead] = (m_ref + log2f(l_tot)) * 0.69314718055994531f;
    } else {
      const long long pidx = static_cast<long long>(gi) * p.H + qhead;
      p.part_ml[pidx * 4] = m_ref;
      p.part_ml[pidx * 4 + 1] = l_tot;
    }
  }
  __syncthreads();
  MLA_PHASE(6);
  // The accumulators are read next; cover the last MFMAs' latency. Each
  // accumulator then passes through an empty asm, so that no copy of it (the
  // compiler's own included) can be placed above the wait.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4 * NW; ++i) asm volatile("" : "+a"(oacc[i]));
  // Epilogue through LDS (the tile stages are free now), 64 heads per
  // round: each wave writes its accumulator blocks of those heads into
  // head rows of 512 floats, then the workgroup stores the rows as one
  // contiguous run, 16 bytes per lane, so every store instruction writes
  // 1 KiB of consecutive output (16-byte pieces of 32 head rows per
  // instruction straight from the accumulators left HBM lines half written).
  // The stores are nontemporal: nothing in this kernel reads them again.
  // D[i][head] of block (c, hb) holds column colbase(4w + c) + 32*((i&15)>>2)
  // + 4*(i>>4) + (i&3); register 4g + m of this lane is i = 8g + 4h + m.
  // A partial (more than one chunk) leaves as fp16 scaled by 2^-E per head
  // row: a first pass over the accumulators records, per wave, the largest
  // magnitude of its 128 columns of each head row (in the weight buffers,
  // free now); the staging pass then takes E from the maximum of the four
  // and writes the scaled values as fp16 rows.
  constexpr int OROW = 2 * 1024 + 16;   // staged fp32 row stride: rows 16 B apart on the banks
  constexpr int OROW16 = 1024 + 16;     // staged fp16 row stride
  static_assert(64 * OROW <= ROPE_OFF, "staged rows must stay below the rotary slots and weight buffers");
  float* hmax = reinterpret_cast<float*>(smem + P_OFF);   // [4 waves][64 rows]
  // One branch-free path for each kind of output.
  auto epilogue = [&](auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
#pragma unroll
    for (int R = 0; R < (NW + 1) / 2; ++R) {
      // this round's accumulators (head blocks 2R and 2R + 1), read once
      float x[2][4][16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        if (2 * R + hh < NW)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x[hh][c][r]) : "a"(oacc[NW * c + 2 * R + hh][r]));
      float sc[2] = {1.f, 1.f};
      if constexpr (PARTIAL) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (2 * R + hh < NW) {
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int r = 0; r < 16; ++r) amax = max2(amax, __builtin_fabsf(x[hh][c][r]));
            amax = max_halves(amax);
            if (h == 0) hmax[64 * w + 32 * hh + l32] = amax;
          }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (2 * R + hh < NW) {
            const int row = 32 * hh + l32;
            const float mx = max2(max2(hmax[row], hmax[64 + row]), max2(hmax[128 + row], hmax[192 + row]));
            int e;
            (void)frexpf(mx, &e);   // mx < 2^e (e = 0 for a zero row)
            sc[hh] = ldexpf(1.f, -e);
            if (w == 0 && h == 0)
              p.part_ml[(static_cast<long long>(gi) * p.H + 32 * (2 * R + hh) + l32) * 4 + 2] = static_cast<float>(e);
          }
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (2 * R + hh < NW) sc[hh] = 1.f / lm[2 * (32 * (2 * R + hh) + l32) + 1];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        if (2 * R + hh < NW)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = colbase(4 * w + c) + 32 * ((2 * g + h) & 3) + 4 * (g >> 1);
              const float* v = &x[hh][c][4 * g];
              const float s = sc[hh];
              if constexpr (PARTIAL) {
                const f16x2 lo = __builtin_convertvector((f32x2{v[0] * s, v[1] * s}), f16x2);
                const f16x2 hi = __builtin_convertvector((f32x2{v[2] * s, v[3] * s}), f16x2);
                *reinterpret_cast<u32x2*>(smem + (32 * hh + l32) * OROW16 + 2 * col) =
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
              } else {
                *reinterpret_cast<f32x4*>(smem + (32 * hh + l32) * OROW + 4 * col) =
                    f32x4{v[0] * s, v[1] * s, v[2] * s, v[3] * s};
              }
            }
      __syncthreads();
      // H = 32 NW, so the row count is a constant of the unrolled round
      const int nrows = min(64, 32 * NW - 64 * R);
      if constexpr (PARTIAL) {
        uint16_t* dst = p.part_o + (static_cast<long long>(gi) * p.H + 64 * R) * DC;
#pragma unroll
        for (int k = 0; k < nrows * (DC / 8) / NTHREADS; ++k) {
          const int idx = tid + NTHREADS * k, row = idx >> 6, piece = idx & 63;
          __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(smem + row * OROW16 + 16 * piece),
                                      reinterpret_cast<f32x4*>(dst + row * DC + 8 * piece));
        }
      } else {
        float* dst = p.o_lat + (static_cast<long long>(b) * p.H + 64 * R) * DC;
#pragma unroll
        for (int k = 0; k < nrows * (DC / 4) / NTHREADS; ++k) {
          const int idx = tid + NTHREADS * k, row = idx >> 7, piece = idx & 127;
          __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(smem + row * OROW + 16 * piece),
                                      reinterpret_cast<f32x4*>(dst + row * DC + 4 * piece));
        }
      }
      __syncthreads();
    }
  };
  if (single) epilogue(std::false_type{});
  else epilogue(std::true_type{});
#ifdef MLA_CLOCK_STAMPS
  if (tid == 0 && blockIdx.x < kStampSlots) {
    unsigned long long* st = g_clock_stamps + 4 * blockIdx.x;
    st[0] = stamp_t0;
    st[1] = __builtin_amdgcn_s_memtime();
    st[2] = stamp_r0;
    st[3] = __builtin_amdgcn_s_memrealtime();
    phase_t[7] = st[1];
    for (int i = 0; i < 8; ++i) g_phase[8 * blockIdx.x + i] = phase_t[i];
  }
#endif
}

// Exact merge of the chunk partials of one (b, head), for sequences with
// more than one chunk: M = max m_j, w_j = 2^(m_j - M),
// o = sum_j w_j O_j / sum_j w_j l_j and lse = (M + log2 sum_j w_j l_j) ln 2,
// with O_j = 2^E_j times its stored fp16 row.
// Up to 64 chunks, lane j of each wave reads (m, l, E) of chunk j, so the
// maximum, weights and denominator come from wave reductions; every thread
// streams 4 columns of every partial once, in groups of 4 (up to four
// chunks) or 16 loads issued before their weights are needed (padding loads
// re-read the last partial and are not added). More chunks take a plain loop.
__global__ __launch_bounds__(128) void combine_chunks(Params p) {
  const int head = blockIdx.x % p.H;
  const int b = blockIdx.x / p.H;
  const int2 pl = p.plan_seq[b];
  const int start = pl.x, n = pl.y;
  if (n <= 1) return;
  const int lane = threadIdx.x & 63;
  const long long so = static_cast<long long>(p.H) * DC;   // partial stride (elements)
  const long long sm = 4LL * p.H;
  const uint16_t* po = p.part_o + (static_cast<long long>(start) * p.H + head) * DC + 4 * threadIdx.x;
  const float* pm = p.part_ml + (static_cast<long long>(start) * p.H + head) * 4;
  auto raw = [&](int j) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(po + j * so)); };
  auto cvt = [](u32x2 u) {
    return f32x4{f16_bits_to_f32(u[0]), f16_bits_to_f32(u[0] >> 16), f16_bits_to_f32(u[1]), f16_bits_to_f32(u[1] >> 16)};
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, den = 0.f;
  if (n <= 64) {
    // GRP partial loads in flight per group (indices past the last chunk
    // re-read it and are not added): one memory latency per group; 4 for up
    // to four chunks, where more would only re-read, else 16
    auto merge = [&](auto grp) {
      constexpr int GRP = decltype(grp)::value;
      u32x2 v[GRP];
#pragma unroll
      for (int g = 0; g < GRP; ++g) v[g] = raw(min(g, n - 1));
      const float m = lane < n ? pm[lane * sm] : -INFINITY;
      const float l = lane < n ? pm[lane * sm + 1] : 0.f;
      const int e = lane < n ? static_cast<int>(pm[lane * sm + 2]) : 0;
      M = wave_reduce(m, [](float a, float c) { return fmaxf(a, c); });
      const float w0 = lane < n ? exp2f(m - M) : 0.f;
      den = wave_reduce(w0 * l, [](float a, float c) { return a + c; });
      const float w = ldexpf(w0, e);   // the weight of the stored (scaled) row
      auto weight = [&](int j) {       // chunk j's weight (j uniform), from its lane
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
      };
      for (int j = 0; j < n; j += GRP) {
        if (j > 0) {
#pragma unroll
          for (int g = 0; g < GRP; ++g) v[g] = raw(min(j + g, n - 1));
        }
#pragma unroll
        for (int g = 0; g < GRP; ++g)
          if (j + g < n) acc += weight(j + g) * cvt(v[g]);
      }
    };
    if (n <= 4) merge(std::integral_constant<int, 4>{});
    else merge(std::integral_constant<int, 16>{});
  } else {
    for (int j = 0; j < n; ++j) M = fmaxf(M, pm[j * sm]);
    for (int j = 0; j < n; ++j) {
      const float w = exp2f(pm[j * sm] - M);
      den += w * pm[j * sm + 1];
      acc += ldexpf(w, static_cast<int>(pm[j * sm + 2])) * cvt(raw(j));
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  __builtin_nontemporal_store(acc * inv,
                              reinterpret_cast<f32x4*>(p.o_lat + (static_cast<long long>(b) * p.H + head) * DC +
                                                       4 * threadIdx.x));
  if (p.lse && threadIdx.x == 0)
    p.lse[b * p.H + head] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

// A launch whose start and end stamp the given events when either is set
// (hipExtLaunchKernel's kernel-timing events, which put no marker command in
// the stream), a plain launch otherwise.
template <typename Kernel>
void launch_timed(Kernel kernel, dim3 grid, int threads, hipStream_t stream, hipEvent_t start, hipEvent_t end,
                  const Params& p) {
  if (start || end)
    hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, start, end, 0, p);
  else
    kernel<<<grid, threads, 0, stream>>>(p);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.cache = static_cast<const uint16_t*>(a.cache);
  p.table = a.block_table;
  p.seq_stride = a.capacity * DW;
  p.bs_log2 = a.block_table ? __builtin_ctz(static_cast<unsigned>(a.block_size)) : 0;
  p.max_blocks = a.max_blocks;
  p.seq_lens = a.seq_lens;
  p.B = a.B;
  p.H = a.H;
  p.grid = a.grid;
  p.splits = a.splits;
  p.sl2 = a.scale * 1.4426950408889634f;
  p.o_lat = a.o_lat;
  p.lse = a.lse;
  p.part_o = reinterpret_cast<uint16_t*>(a.part_o);   // fp16 partials on this path
  p.part_ml = a.part_ml;
  p.plan_seq = a.plan_seq;
  p.indices = a.indices;
  p.topk = a.topk;
  p.qpt = a.qpt;
  const dim3 grid(a.grid);
  const int pm = a.indices ? (a.block_table ? GATHER_PAGED : GATHER_CONTIG)
                           : (!a.block_table ? CONTIG : (a.block_size >= 8 ? PAGED8 : PAGED_SMALL));
  // with one workgroup per sequence every sequence has a single chunk and no
  // merge runs; the kernel is then the call's last
  const bool merge = a.grid > a.B;
  hipEvent_t k_end = a.t_kernel_end ? a.t_kernel_end : (merge ? nullptr : a.t_call_end);
#define MLA_ATTN_LAUNCH(NW)                                                                                     \
  if (pm == CONTIG) launch_timed(attn_mfma_kernel<NW, CONTIG>, grid, NTHREADS, stream, a.t_start, k_end, p);     \
  else if (pm == PAGED8) launch_timed(attn_mfma_kernel<NW, PAGED8>, grid, NTHREADS, stream, a.t_start, k_end, p); \
  else if (pm == PAGED_SMALL)                                                                                   \
    launch_timed(attn_mfma_kernel<NW, PAGED_SMALL>, grid, NTHREADS, stream, a.t_start, k_end, p);               \
  else if (pm == GATHER_CONTIG)                                                                                 \
    launch_timed(attn_mfma_kernel<NW, GATHER_CONTIG>, grid, NTHREADS, stream, a.t_start, k_end, p);             \
  else launch_timed(attn_mfma_kernel<NW, GATHER_PAGED>, grid, NTHREADS, stream, a.t_start, k_end, p);
  switch (a.H / 32) {
    case 1: MLA_ATTN_LAUNCH(1) break;
    case 2: MLA_ATTN_LAUNCH(2) break;
    case 3: MLA_ATTN_LAUNCH(3) break;
    case 4: MLA_ATTN_LAUNCH(4) break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_ATTN_LAUNCH
  if (merge) launch_timed(combine_chunks, dim3(a.B * a.H), 128, stream, nullptr, a.t_call_end, p);
  else if (a.t_kernel_end && a.t_call_end) {
    const hipError_t e = hipEventRecord(a.t_call_end, stream);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace mla

#ifdef MLA_CLOCK_STAMPS
// Copy the stamps of workgroups 0..n-1 of the last attention launch ([n][4]:
// start cycles, end cycles, start real time, end real time) to host memory.
extern "C" int mla_clock_stamps(unsigned long long* host_dst, int n) {
  if (n < 0 || n > mla::kStampSlots) return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(mla::g_clock_stamps),
                                              sizeof(unsigned long long) * 4 * n, 0, hipMemcpyDeviceToHost));
}
// Zero every stamp (then only the workgroups of the next launch that have a
// chunk write theirs).
extern "C" int mla_clock_stamps_reset(void) {
  void* a = nullptr;
  void* b = nullptr;
  hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(mla::g_clock_stamps));
  if (e == hipSuccess) e = hipGetSymbolAddress(&b, HIP_SYMBOL(mla::g_phase));
  if (e == hipSuccess) e = hipMemset(a, 0, sizeof(mla::g_clock_stamps));
  if (e == hipSuccess) e = hipMemset(b, 0, sizeof(mla::g_phase));
  return static_cast<int>(e);
}
// The phase stamps of workgroups 0..n-1 ([n][8] shader-clock values) of the
// last attention launch.
extern "C" int mla_phase_stamps(unsigned long long* host_dst, int n) {
  if (n < 0 || n > mla::kStampSlots) return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(mla::g_phase),
                                              sizeof(unsigned long long) * 8 * n, 0, hipMemcpyDeviceToHost));
}
#endif
