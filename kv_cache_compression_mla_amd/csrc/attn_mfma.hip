// Latent-space MLA decode attention on gfx950 bf16 MFMA.
//
// Every query head attends directly against the shared latent cache: the
// absorbed query q(i) = [W_UK(i)^T q_C(i) ; q_R(i)] is dotted with whole
// 576-wide rows [c_u ; kR_u], and the softmax weights combine the latents
// c_u themselves ("Understanding MLA" (Dong), section 4: the key
// up-projection moves onto the query; aicassindra MLA explainer, "End-to-end
// flow": content and rotary dot products summed, softmax over all history).
//
// Work decomposition: one workgroup = one sequence x one context chunk x all
// H heads, one wave per 32 heads. The heads that share a latent row form a
// dense contraction:
//   S^T[row][head] = K_tile[row][0:576] . Q^T[0:576][head]     (MFMA 32x32x16)
//   O^T[col][head] += V_tile^T[col][rows] . P[rows][head]      (MFMA 32x32x16)
// with V_tile = K_tile[:, 0:512]. A wave keeps its query block (32 heads x
// 576, bf16) in VGPRs and its O^T accumulator (512 x 32 fp32) in AGPRs for
// the whole chunk. The score contraction runs as two interleaved
// accumulation chains (even and odd 16-column steps) so that consecutive
// MFMAs are independent.
//
// Memory path: each 32-row tile is copied HBM -> LDS once per workgroup by
// LDS-DMA (global_load_lds, 16 B per lane, one 1 KiB row latent per copy),
// four stages deep, so nothing is staged in registers. In LDS the latent
// rows sit at a 1040-byte stride and the rotary parts are packed 128 B per
// row with an XOR swizzle of their 16-byte chunks. The score operand is read
// with ds_read_b128 (lanes walk rows); the value operand, whose reduction
// index is the row, is read transposed with ds_read_b64_tr_b16 from the same
// row-major copy. A value block of 32 columns covers four runs of 8 columns
// 32 apart, which makes the transposed reads of 32 lanes tile all 64 banks;
// both read patterns are bank-conflict free and every address is one
// per-lane base plus a compile-time offset.
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
// Context splits: a workgroup covers rows [s*chunk, min((s+1)*chunk, L_b)).
// With more than one split it writes unnormalised (O, m, l) partials, merged
// exactly by attn_combine.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int DC = 512;               // latent width
constexpr int DW = 576;               // row width (latent + rotary key)
constexpr int TILE = 32;              // rows per stage
constexpr int LROW = 1040;            // LDS stride of a latent row (1024 + 16)
constexpr int LAT_BYTES = TILE * LROW;          // 33280
constexpr int STAGE = LAT_BYTES + TILE * 128;   // 37376
constexpr int NSTAGE = 4;
constexpr int NTHREADS = 256;
constexpr int DMA_PER_WAVE = 9;       // 8 latent rows + 1 rotary block per tile
// Fast pass: a head's reference maximum is its first tile's maximum. A later
// tile exceeding it by more than this (log2 units) sends the workgroup to the
// exact two-pass fallback; otherwise probabilities stay in (0, 2^32].
constexpr float REF_GAP = 32.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct Params {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ cache;
  const int32_t* __restrict__ table;
  long long seq_stride;   // contiguous: capacity * DW elements
  int bs_log2, max_blocks;
  const int32_t* __restrict__ seq_lens;
  int H, chunk, splits;
  float sl2;              // softmax scale * log2(e)
  float* o_lat;
  float* lse;
  float* part_o;
  float* part_ml;
};

// XOR swizzle of the 16-byte chunks of a packed 128-byte rotary row: 16
// lanes reading one chunk of 16 rows hit distinct bank groups.
__device__ __forceinline__ int rope_sw(int r) { return (r >> 1) & 7; }

// First column of value block cb: blocks hold columns
// colbase + {0..7} + 32 * {0..3}.
__host__ __device__ constexpr int colbase(int cb) { return 8 * (cb % 4) + 128 * (cb / 4); }

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
template <bool PAGED>
__device__ __forceinline__ const uint16_t* row_ptr(const Params& p, int b, int u) {
  if constexpr (!PAGED) {
    return p.cache + b * p.seq_stride + static_cast<long long>(u) * DW;
  } else {
    const const_i32* tab = (const const_i32*)(p.table);
    const int blk = tab[b * p.max_blocks + (u >> p.bs_log2)];
    return p.cache + ((static_cast<long long>(blk) << p.bs_log2) + (u & ((1 << p.bs_log2) - 1))) * DW;
  }
}

// One LDS-DMA copy: every lane moves 16 bytes from its global address to LDS
// at lds_base + 16 * lane. Written as inline asm so that the compiler does not
// add its own (conservative, vmcnt(0)) waits in front of later LDS reads; the
// kernel waits for these copies explicitly (wait_vmcnt + barrier). The copy
// has no register result, and its address operands are read at issue.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(gptr) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Issue this wave's 9 LDS-DMA copies of tile rows [r0, r0+32) into the stage
// at LDS address `st`: the latents of rows 8w..8w+7 (1 KiB each, straight)
// and the rotary parts of the same 8 rows (128 B each, one copy). Rows at or
// past row_end are replaced by row_end-1 (a real row, later masked out of the
// softmax), so no invalid address is ever read. w, r0, row_end are uniform.
template <bool PAGED>
__device__ __forceinline__ void issue_tile(const Params& p, uint32_t st, int b, int r0, int row_end,
                                           int w, int lane) {
  const uint16_t* rp[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rp[k] = row_ptr<PAGED>(p, b, min(r0 + 8 * w + k, row_end - 1));
#pragma unroll
  for (int k = 0; k < 8; ++k) dma16(rp[k] + 8 * lane, st + (8 * w + k) * LROW);
  // rotary block: lane -> row 8w + (lane >> 3), chunk (lane & 7) ^ rope_sw(row)
  const int j = lane >> 3;
  const uint16_t* mine = rp[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) mine = (j == k) ? rp[k] : mine;
  const int c = (lane & 7) ^ rope_sw(8 * w + j);
  dma16(mine + DC + 8 * c, st + LAT_BYTES + w * 1024);
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// MFMA instructions issued from inline asm are invisible to the compiler's
// hazard tracking. Where an operand is produced by the VALU (the zero
// operand, the packed probabilities) the asm carries the VALU-write to
// MFMA-read wait states itself; where the VALU reads an MFMA result next, the
// wait states follow the MFMA inside the same asm statement, so no read can
// be scheduled in between. All other operands come from memory loads, whose
// completion the compiler's counter waits cover; a CPU test scans the
// compiled ISA for every VALU write close before an MFMA that reads it.
#define MLA_MFMA_PRE "s_nop 4\n\t"
#define MLA_MFMA_POST "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"

// acc = 0 * 0 + 0: clears an accumulator block through the MFMA unit.
__device__ __forceinline__ void mfma_zero(f32x16& acc, const bf16x8& zero8) {
  asm volatile(MLA_MFMA_PRE "v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero8));
}

template <int NW, bool PAGED>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(Params p) {
  __shared__ __align__(1024) char smem[NSTAGE * STAGE];
  __shared__ int wg_flag;
  const uint32_t smem_lds = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int s_idx = blockIdx.x % p.splits;
  const int b = blockIdx.x / p.splits;

  const int L = p.seq_lens[b];
  const int row_begin = s_idx * p.chunk;
  const int row_end = min(row_begin + p.chunk, L);
  const bool active = w < NW;
  const int head = 32 * w + l32;

  if (row_begin >= row_end) {
    // Nothing to attend in this chunk. With splits > 1 the combine kernel
    // skips it; with a single split the sequence is empty.
    if (p.splits == 1 && active) {
      float* o = p.o_lat + (static_cast<long long>(b) * p.H + head) * DC;
      for (int c = h * 256; c < h * 256 + 256; c += 4)
        *reinterpret_cast<f32x4*>(o + c) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p.lse && h == 0) p.lse[b * p.H + head] = -INFINITY;
    }
    return;
  }
  const int ntiles = (row_end - row_begin + TILE - 1) / TILE;

  // Query of this lane's head in MFMA B-operand order: step s, half h holds
  // columns 16s + 8h .. 16s + 8h + 7.
  bf16x8 qreg[36];
  if (active) {
    const uint16_t* qp = p.q + (static_cast<long long>(b) * p.H + head) * DW + 8 * h;
#pragma unroll
    for (int s = 0; s < 36; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  const bf16x8 zero8 = {};
  f32x16 oacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) mfma_zero(oacc[i], zero8);
  float m_ref = -INFINITY;   // reference maximum, log2 units
  float l_run = 0.f;         // this lane's partial sum (its 16 of each 32 rows)

  // Per-lane LDS bases inside a stage; every other part of an operand address
  // is a compile-time immediate of the unrolled loops below.
  //  score operand: row l32, latent chunk 2s + h at 16 * (2s + h)
  const int qk_base = l32 * LROW + 16 * h;
  //  rotary part of row l32: chunk c' at 16 * (c' ^ rope_sw(l32))
  const int rp_base = LAT_BYTES + l32 * 128;
  const int rp_sw = rope_sw(l32);
  //  value operand, transposed read: in its 16-lane group a lane supplies row
  //  16t + 8k + 4*(g16>>1) + tr_e, 8 bytes at column colbase(cb) + 32*tr_q + 4*(g16&1)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_base = (4 * (g16 >> 1) + (i16 >> 2)) * LROW + 64 * (i16 & 3) + 8 * (g16 & 1);

  // mode 0: fast pass (first-tile reference); mode 1: scores only, exact
  // maximum (fallback); mode 2: full pass against that maximum (fallback).
  int mode = 0;
  for (;;) {
    // Prologue: tiles 0..NSTAGE-2 in flight. Then wait for everything issued
    // so far (the query and these copies) so that no vector-memory wait stays
    // pending inside the loop: the loop's waits are the explicit ones below.
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j)
      if (j < ntiles) issue_tile<PAGED>(p, smem_lds + j * STAGE, b, row_begin + j * TILE, row_end, w, lane);
    wait_vmcnt<0>();
    bool grew = false;
    float m_seen = -INFINITY;

    for (int it = 0; it < ntiles; ++it) {
      // Tile `it` was issued NSTAGE-1 iterations ago; later tiles may still fly.
      const int later = min(ntiles - 1 - it, NSTAGE - 2);
      if (later >= 2) wait_vmcnt<2 * DMA_PER_WAVE>();
      else if (later == 1) wait_vmcnt<DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      block_barrier();
      if (it + NSTAGE - 1 < ntiles)
        issue_tile<PAGED>(p, smem_lds + ((it + NSTAGE - 1) % NSTAGE) * STAGE, b,
                          row_begin + (it + NSTAGE - 1) * TILE, row_end, w, lane);
      if (!active) continue;

      const char* st = smem + (it % NSTAGE) * STAGE;
      const int nv = min(TILE, row_end - (row_begin + it * TILE));

      // ---- scores: S^T[row][head] over all 576 columns ----
      // Two accumulation chains (even / odd steps); operand reads run two
      // steps ahead of the MFMA that consumes them.
      auto qk_operand = [&](int s) -> bf16x8 {
        const char* ap = (s < 32) ? st + qk_base + 32 * s
                                  : st + rp_base + 16 * ((2 * (s - 32) + h) ^ rp_sw);
        return *reinterpret_cast<const bf16x8*>(ap);
      };
      f32x16 sacc0, sacc1;
      bf16x8 a0 = qk_operand(0), a1 = qk_operand(1);
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        const bf16x8 a2 = (s + 2 < 36) ? qk_operand(s + 2) : a0;
        if (s == 0) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc0) : "v"(a0), "v"(qreg[s]));
        } else if (s == 1) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc1) : "v"(a0), "v"(qreg[s]));
        } else if (s < 35) {
          if (s & 1)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc1) : "v"(a0), "v"(qreg[s]));
          else
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc0) : "v"(a0), "v"(qreg[s]));
        } else {
          // last step: the VALU reads both chains next
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0" MLA_MFMA_POST
                       : "+v"(sacc1), "+v"(sacc0) : "v"(a0), "v"(qreg[s]));
        }
        a0 = a1;
        a1 = a2;
      }
      f32x16 sacc = sacc0 + sacc1;

      // ---- softmax weights (base 2) against the reference maximum ----
      // Scores are scaled once (x = s * scale * log2 e); the maximum and the
      // exponents use the same rounded x, so a row at the reference gets
      // weight exactly 1.
      sacc *= p.sl2;
      if (nv < TILE) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * h + (r & 3) >= nv) sacc[r] = -INFINITY;
      }
      float tmax = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sacc[r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (mode == 1) {
        m_seen = fmaxf(m_seen, tmax);
        continue;
      }
      if (mode == 0) {
        if (it == 0) m_ref = tmax;
        else grew = grew || (tmax > m_ref + REF_GAP);
      }
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = __builtin_amdgcn_exp2f(sacc[r] - m_ref);
        psum += sacc[r];
      }
      l_run += psum;
      bf16x8 pb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          bf16x2 v2 = __builtin_convertvector((f32x2{sacc[8 * t + 2 * k], sacc[8 * t + 2 * k + 1]}), bf16x2);
          pb[t][2 * k] = v2[0];
          pb[t][2 * k + 1] = v2[1];
        }
      // P was just written by the VALU and is read by MFMAs next (VALU-write
      // to MFMA-read wait states, tied to the operands).
      asm volatile("s_nop 4" : "+v"(pb[0]), "+v"(pb[1]));

      // ---- O^T[col][head] += V^T P ----
      // Steps run t-major (all 16 column blocks for rows 0-15, then rows
      // 16-31) so that the two MFMAs into one accumulator are 16 apart; the
      // transposed operand reads run two steps ahead.
      auto pv_operand = [&](int cb, int t) -> bf16x8 {
        const char* a = st + tr_base + (16 * LROW) * t + 2 * colbase(cb);
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * LROW));
        return __builtin_bit_cast(bf16x8, (s16x8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
      };
      bf16x8 v0 = pv_operand(0, 0), v1 = pv_operand(1, 0);
#pragma unroll
      for (int step = 0; step < 32; ++step) {
        const int t = step >> 4, cb = step & 15;
        const bf16x8 v2 = (step + 2 < 32) ? pv_operand((step + 2) & 15, (step + 2) >> 4) : v0;
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(oacc[cb]) : "v"(v0), "v"(pb[t]));
        v0 = v1;
        v1 = v2;
      }
    }

    if (mode == 2) break;
    if (mode == 1) {
      // exact maximum known: redo the chunk against it
      m_ref = m_seen;
      l_run = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) mfma_zero(oacc[i], zero8);
      mode = 2;
      __syncthreads();
      continue;
    }
    // mode 0 done: did any head in the workgroup outgrow its reference?
    if (tid == 0) wg_flag = 0;
    __syncthreads();
    if (active && __builtin_amdgcn_ballot_w64(grew) != 0 && lane == 0) wg_flag = 1;
    __syncthreads();
    if (wg_flag == 0) break;
    mode = 1;
    __syncthreads();
  }

  if (!active) return;
  // The accumulators are read next; cover the last MFMAs' latency.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (p.splits == 1) ? 1.f / l_tot : 1.f;
  float* o = (p.splits == 1)
                 ? p.o_lat + (static_cast<long long>(b) * p.H + head) * DC
                 : p.part_o + ((static_cast<long long>(b) * p.splits + s_idx) * p.H + head) * DC;
  // D[i][head] of block cb holds column colbase(cb) + 32*((i&15)>>2) + 4*(i>>4) + (i&3);
  // register 4g + m of this lane is i = 8g + 4h + m.
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x[r]) : "a"(oacc[cb][r]));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = colbase(cb) + 32 * ((2 * g + h) & 3) + 4 * (g >> 1);
      *reinterpret_cast<f32x4*>(o + col) =
          f32x4{x[4 * g] * inv, x[4 * g + 1] * inv, x[4 * g + 2] * inv, x[4 * g + 3] * inv};
    }
  }
  if (h == 0) {
    if (p.splits == 1) {
      if (p.lse) p.lse[b * p.H + head] = (m_ref + log2f(l_tot)) * 0.69314718055994531f;
    } else {
      const long long pidx = (static_cast<long long>(b) * p.splits + s_idx) * p.H + head;
      p.part_ml[pidx * 2] = m_ref;
      p.part_ml[pidx * 2 + 1] = l_tot;
    }
  }
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
  p.H = a.H;
  p.chunk = a.chunk;
  p.splits = a.splits;
  p.sl2 = a.scale * 1.4426950408889634f;
  p.o_lat = a.o_lat;
  p.lse = a.lse;
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  const dim3 grid(a.B * a.splits);
  const bool paged = a.block_table != nullptr;
#define MLA_ATTN_LAUNCH(NW)                                                          \
  if (paged) attn_mfma_kernel<NW, true><<<grid, NTHREADS, 0, stream>>>(p);           \
  else attn_mfma_kernel<NW, false><<<grid, NTHREADS, 0, stream>>>(p);
  switch (a.H / 32) {
    case 1: MLA_ATTN_LAUNCH(1) break;
    case 2: MLA_ATTN_LAUNCH(2) break;
    case 3: MLA_ATTN_LAUNCH(3) break;
    case 4: MLA_ATTN_LAUNCH(4) break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
