// Causal prefill attention in the materialised ("training") form.
//
// The step on the other side of the cache: T new tokens per sequence attend
// causally over the cached rows, with every head's keys and values rebuilt
// from the latents, K(i)_u = [W_UK(i) c_u ; k_R,u] and V(i)_u = W_UV(i) c_u
// ("Understanding MLA" (Dong), phase B and D, and sections 5-6 on the
// training form; llm-arch-kb "Multi-Head Latent Attention", section 3
// sketch, which expands the latent and runs ordinary attention over
// [B, H, T, T] scores). The expansion runs before this kernel (a GEMM over
// every stored row); here query token t of sequence b, at position
// p = seq_lens[b] - T + t, takes
//   s(u) = scale * (q_C . K_nope(u) + q_R . k_R(u))   u = 0..p
//   o    = sum_u softmax(s)(u) V(u),  lse = ln sum_u exp s(u).
//
// MFMA kernel (bf16, d_h = d_v = 128, d_R = 64): one workgroup of four waves
// per (sequence, head, 128-query tile), 32 queries per wave. 32-key tiles of
// the expanded keys, the rotary keys and the transposed values go HBM -> LDS
// by LDS-DMA through a ring of four buffers (fetched three tiles ahead, one
// barrier per tile; 80 KiB, two workgroups per CU) and are shared by the four
// waves. Per tile and wave:
//   S^T = K . Q^T    (32 keys x 32 queries, 12 MFMA 32x32x16 over 192 features)
//   O^T += V^T . P^T (128 d_v x 32 queries, 8 MFMA over 32 keys)
// with the softmax of a query held in the lane that owns its column. The
// weights use a fixed per-query reference (rescaled only when a tile's
// maximum exceeds it by 2^16), so O is written only by MFMA in the tile
// loop; each weight is one fma and the hardware exp2, and the packed bf16
// weights trade one pair of words between lane halves to reach the value
// MFMA's key order.
#include "mla_internal.hpp"

namespace mla {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int PF_NQB = 1;    // 32-query MFMA blocks per wave (two do not fit in registers without spills)
constexpr int PF_NW = 4;     // waves per workgroup
constexpr int PF_NBUF = 4;   // tile buffers in the copy ring
constexpr int KT = 32;         // keys per tile
constexpr int DH = 128, DR = 64, DV = 128;
constexpr int DQ = DH + DR;    // query / key width
constexpr int SK = DQ / 16;    // MFMA k-steps of the scores
// LDS (16-byte slots) of one tile buffer: expanded keys 32 x 16 chunks,
// rotary keys 32 x 8 chunks, transposed values 128 x 4 chunks; XOR swizzles
// keep each group of 16 lanes of an MFMA operand read on distinct banks.
constexpr int KN_SLOTS = KT * 16;
constexpr int KR_SLOTS = KT * 8;
constexpr int VT_SLOTS = DV * 4;
constexpr int BUF_SLOTS = KN_SLOTS + KR_SLOTS + VT_SLOTS;   // 20 KiB

__device__ __forceinline__ int kn_slot(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ __forceinline__ int kr_slot(int r, int c) { return KN_SLOTS + r * 8 + (c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int vt_slot(int m, int c) { return KN_SLOTS + KR_SLOTS + m * 4 + (c ^ ((m >> 2) & 3)); }

// Storage row of row u of sequence b (the expanded keys use the same index)
// and the column of the transposed values.
__device__ __forceinline__ long long store_row(const PrefillArgs& a, int b, int u) {
  if (a.block_table == nullptr) return static_cast<long long>(b) * a.capacity + u;
  const int blk = a.block_table[b * a.max_blocks + u / a.block_size];
  return static_cast<long long>(blk) * a.block_size + u % a.block_size;
}
__device__ __forceinline__ long long vt_col(const PrefillArgs& a, int b, int u) {
  if (a.block_table == nullptr) return static_cast<long long>(b) * a.vt_seq + u;
  return store_row(a, b, u);
}
// LDS-DMA: each lane moves 16 bytes from its address to LDS at lds + 16 *
// lane. Inline asm so that the compiler adds none of its own waits; the
// kernel waits for the copies (vmcnt(0)) before the barrier that publishes
// the tile. The copy has no register result; its operands are read at issue.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(gptr));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// NW waves per workgroup, NQB 32-query MFMA blocks per wave, NBUF tile
// buffers in the copy ring (tiles are fetched NBUF - 1 ahead).
template <bool PAGED, int NW, int NQB, int NBUF>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a, int bs_log2) {
  constexpr int QW = 32 * NQB;   // queries per wave
  constexpr int QT = NW * QW;    // queries per workgroup
  constexpr int KN_CP = KN_SLOTS / 64 / NW, KR_CP = KR_SLOTS / 64 / NW, VT_CP = VT_SLOTS / 64 / NW;
  constexpr int PW = KN_CP + KR_CP + VT_CP;   // copies per wave per tile
  static_assert(KN_SLOTS % (64 * NW) == 0 && KR_SLOTS % (64 * NW) == 0 && VT_SLOTS % (64 * NW) == 0, "copy split");
  __shared__ __align__(16) u32x4 lds[NBUF * BUF_SLOTS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
  // consecutive ids (the query tiles of one sequence and head, which read
  // the same keys and values) share an XCD and its L2.
  const int nb = gridDim.x, per = nb / 8;
  const int bid = blockIdx.x;
  const int id = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
  const int ntq = (a.T + QT - 1) / QT;
  const int qt = id % ntq;
  const int head = (id / ntq) % a.H;
  const int b = id / (ntq * a.H);

  const int L = a.seq_lens[b];
  const int base = L - a.T;                  // position of token 0
  const int t0 = qt * QT;
  const int tw0 = t0 + QW * w;               // this wave's first query
  const bool wave_live = tw0 < a.T;
  const int key_end = base + min(t0 + QT, a.T);          // keys [0, key_end) of the workgroup
  const int wave_qmin = base + tw0;                       // positions of this wave's queries
  const int wave_qmax = base + min(tw0 + QW, a.T) - 1;
  const float sl2 = a.scale * 1.4426950408889634f;

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kx = static_cast<const uint16_t*>(a.K);
  const uint16_t* Vt = static_cast<const uint16_t*>(a.Vt);
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache);
  const int D = a.d_c + a.d_R;
  const long long kstride = static_cast<long long>(a.H) * DH;   // expanded-key row length

  // Query of each lane (column l32 of query block qb) in B-operand order;
  // queries past T repeat the last one and are not stored.
  bf16x8 qr[NQB][SK];
  int qpos[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int te = min(tw0 + 32 * qb + l32, a.T - 1);
    qpos[qb] = base + te;
    const uint16_t* qp = q + ((static_cast<long long>(b) * a.T + te) * a.H + head) * DQ + 8 * h;
#pragma unroll
    for (int s = 0; s < SK; ++s) qr[qb][s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  f32x16 oacc[NQB][4];
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) oacc[qb][j] = f32x16{};
  }

  // One tile by LDS-DMA: expanded keys (4 rows per copy), rotary keys (8 rows
  // per copy) and transposed values (16 value rows of 32 keys per copy), each
  // lane fetching the chunk its destination slot holds under the swizzle.
  // Key rows past key_end fetch row key_end - 1 and value chunks past it the
  // last chunk holding a valid key (real data in bounds; the keys are masked
  // and the values zeroed before use).
  const uint32_t lds0 = lds_addr(lds);
  const int last8 = ((key_end - 1) >> 3) << 3;
  // Paged: the (at most 4, block_size >= 8) blocks of a 32-key tile, read
  // as scalar loads (through the constant address space, counted by
  // lgkmcnt) so that the explicit vmcnt waits on the copies stay exact.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  int tb[4] = {0, 0, 0, 0};
  int tb0 = 0;
  auto tile_blocks = [&](int u0) {
    if constexpr (PAGED) {
      const const_i32* tab = (const const_i32*)(a.block_table) + static_cast<long long>(b) * a.max_blocks;
      tb0 = u0 >> bs_log2;
      const int lastb = (key_end - 1) >> bs_log2;
#pragma unroll
      for (int i = 0; i < 4; ++i) tb[i] = tab[min(tb0 + i, lastb)];
    }
  };
  // storage row of key u (u0 <= u < u0 + 32, u < key_end) of this tile
  auto srow = [&](int u) -> long long {
    if constexpr (PAGED) {
      const int i = (u >> bs_log2) - tb0;
      const int blk = i == 0 ? tb[0] : i == 1 ? tb[1] : i == 2 ? tb[2] : tb[3];
      return (static_cast<long long>(blk) << bs_log2) + (u & ((1 << bs_log2) - 1));
    } else {
      return static_cast<long long>(b) * a.capacity + u;
    }
  };
  auto copy_tile = [&](int buf, int u0) {
    const uint32_t bb = lds0 + buf * BUF_SLOTS * 16;
    tile_blocks(u0);
#pragma unroll
    for (int k = 0; k < KN_CP; ++k) {
      const int cp = w + NW * k;
      const int r = 4 * cp + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const int u = min(u0 + r, key_end - 1);
      dma16(Kx + srow(u) * kstride + head * DH + 8 * c,
            __builtin_amdgcn_readfirstlane(bb + cp * 1024));
    }
#pragma unroll
    for (int k = 0; k < KR_CP; ++k) {
      const int cp = w + NW * k;
      const int r = 8 * cp + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int u = min(u0 + r, key_end - 1);
      dma16(cache + srow(u) * D + a.d_c + 8 * c,
            __builtin_amdgcn_readfirstlane(bb + KN_SLOTS * 16 + cp * 1024));
    }
#pragma unroll
    for (int k = 0; k < VT_CP; ++k) {
      const int cp = w + NW * k;
      const int mrow = 16 * cp + (lane >> 2);
      const int c = (lane & 3) ^ ((mrow >> 2) & 3);
      const int u = min(u0 + 8 * c, last8);
      const long long col = PAGED ? srow(u) : static_cast<long long>(b) * a.vt_seq + u;
      dma16(Vt + (static_cast<long long>(head) * DV + mrow) * a.vt_ld + col,
            __builtin_amdgcn_readfirstlane(bb + (KN_SLOTS + KR_SLOTS) * 16 + cp * 1024));
    }
  };
  // Before computing tile it: this wave's copies of tile it are done
  // (later tiles' copies may still be in flight), then a barrier publishes
  // every wave's copies and frees the buffer of tile it - 1 for tile
  // it + NBUF - 1. The last tile zeroes its value columns past key_end.
  auto wait_copies = [&](int later) {
    if (later >= 3) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * PW) : "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * PW) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto sync_tile = [&](int it, int ntiles) {
    wait_copies(min(NBUF - 2, ntiles - 1 - it));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (it + NBUF - 1 < ntiles) copy_tile((it + NBUF - 1) % NBUF, (it + NBUF - 1) * KT);
    if (it == ntiles - 1 && (it + 1) * KT > key_end) {
      char* Bc = reinterpret_cast<char*>(lds + (it % NBUF) * BUF_SLOTS);
      const int kv = key_end - it * KT;   // valid keys in this tile
      for (int e = tid; e < DV * KT; e += 64 * NW) {
        const int mrow = e / KT, key = e % KT;
        if (key >= kv)
          *reinterpret_cast<uint16_t*>(Bc + vt_slot(mrow, key >> 3) * 16 + (key & 7) * 2) = 0;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // Scores of one tile (S^T = K . Q^T), scaled to log2 units and masked;
  // mx: each query's largest score in the tile.
  f32x16 sacc[NQB];
  float mx[NQB];
  // The 12 k-steps run as two interleaved accumulation chains (even and odd
  // steps, summed at the end) so that consecutive MFMAs do not wait on each
  // other's results, with the key operands read PF steps ahead.
  constexpr int PF = 4;
  auto scores = [&](int buf, int u0) {
    const u32x4* B = lds + buf * BUF_SLOTS;
    auto operand = [&](int s) -> u32x4 {
      return s < DH / 16 ? B[kn_slot(l32, 2 * s + h)] : B[kr_slot(l32, 2 * (s - DH / 16) + h)];
    };
    f32x16 sodd[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      sacc[qb] = f32x16{};
      sodd[qb] = f32x16{};
    }
    u32x4 ops[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ops[i] = operand(i);
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      const u32x4 av = ops[s % PF];
      if (s + PF < SK) ops[s % PF] = operand(s + PF);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (s & 1)
          sodd[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), qr[qb][s], sodd[qb],
                                                             0, 0, 0);
        else
          sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), qr[qb][s], sacc[qb],
                                                             0, 0, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) sacc[qb] += sodd[qb];
    const bool need_mask = u0 + KT - 1 > wave_qmin;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // lane (h, l32) holds query l32's raw scores of keys 8(r/4) + 4h + r%4;
      // the maximum is taken on raw scores (the scale is positive) and
      // scaled once
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (u0 + 8 * (r >> 2) + 4 * h + (r & 3) > qpos[qb]) sacc[qb][r] = -INFINITY;
      }
      float x = sacc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, sacc[qb][r]);
      mx[qb] = fmaxf(x, __shfl_xor(x, 32)) * sl2;
    }
  };
  // Softmax weights against the reference m (set from the first tile that
  // has a key; O is still zero then), the normaliser, and O^T += V^T . P^T.
  // The B operand of k-step kk needs keys 16kk + 8h .. + 7 in lane half h;
  // the score registers hold keys 16kk + 4h + 0..3 and 16kk + 8 + 4h + 0..3,
  // so the halves trade one pair of packed words.
  auto weights_and_values = [&](int buf) {
    const u32x4* B = lds + buf * BUF_SLOTS;
    bf16x8 pk[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (m[qb] == -INFINITY) m[qb] = mx[qb];
      const float mref = m[qb] == -INFINITY ? 0.f : m[qb];   // no key yet: every p is 0
      // weight 2^(s * sl2 - mref): one fma and the hardware exp2 (masked
      // scores are -inf and give 0; weights are at most 2^REF_SLACK)
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], sl2, -mref));
        sacc[qb][r] = pv;
        sum += pv;
      }
      l[qb] += sum + __shfl_xor(sum, 32);
      auto pk2 = [](float a, float b) -> uint32_t {   // nearest-even bf16 pair (v_cvt_pk_bf16_f32)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
      };
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint32_t w0 = pk2(sacc[qb][8 * kk + 0], sacc[qb][8 * kk + 1]);
        const uint32_t w1 = pk2(sacc[qb][8 * kk + 2], sacc[qb][8 * kk + 3]);
        const uint32_t w2 = pk2(sacc[qb][8 * kk + 4], sacc[qb][8 * kk + 5]);
        const uint32_t w3 = pk2(sacc[qb][8 * kk + 6], sacc[qb][8 * kk + 7]);
        const uint32_t s0 = __shfl_xor(h ? w0 : w2, 32);
        const uint32_t s1 = __shfl_xor(h ? w1 : w3, 32);
        const u32x4 pw = h ? u32x4{s0, s1, w2, w3} : u32x4{w0, w1, s0, s1};
        pk[qb][kk] = __builtin_bit_cast(bf16x8, pw);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 av = B[vt_slot(32 * j + l32, 2 * kk + h)];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          oacc[qb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pk[qb][kk],
                                                                oacc[qb][j], 0, 0, 0);
      }
    }
  };

  // The reference stays fixed while every tile's maximum is within 2^16 of
  // it (weights up to 2^16 are exact in float32 and in bf16's range), so the
  // accumulators are only ever written by MFMA in the tile loop. A tile that
  // exceeds it leaves the loop, rescales O and l to the new maximum and
  // continues: a rare event after the first tiles.
  constexpr float REF_SLACK = 16.f;
  if (key_end > 0) {
    const int ntiles = (key_end + KT - 1) / KT;
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < ntiles) copy_tile(t, t * KT);
    int it = 0;
    while (it < ntiles) {
      bool rescale = false;
#pragma unroll 1
      for (; it < ntiles; ++it) {
        sync_tile(it, ntiles);
        if (wave_live && it * KT <= wave_qmax) {   // else every key of the tile follows this wave's queries
          scores(it % NBUF, it * KT);
          bool over = false;
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) over |= m[qb] != -INFINITY && mx[qb] > m[qb] + REF_SLACK;
          if (__any(over)) {
            rescale = true;
            break;
          }
          weights_and_values(it % NBUF);
        }
      }
      if (rescale) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float m_new = fmaxf(m[qb], mx[qb]);
          const float alpha = m[qb] == -INFINITY ? 0.f : exp2f(m[qb] - m_new);
          l[qb] *= alpha;
#pragma unroll
          for (int j = 0; j < 4; ++j) oacc[qb][j] *= alpha;
          m[qb] = m_new;
        }
        weights_and_values(it % NBUF);
        ++it;
      }
    }
  }

  // O^T: lane (h, l32) holds d_v rows 32j + 8(r/4) + 4h + r%4 of query l32
  uint16_t* o = static_cast<uint16_t*>(a.o);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int t = tw0 + 32 * qb + l32;
    if (!wave_live || t >= a.T) continue;
    const float inv = l[qb] > 0.f ? 1.f / l[qb] : 0.f;
    uint16_t* orow = o + ((static_cast<long long>(b) * a.T + t) * a.H + head) * DV;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * j + 8 * g + 4 * h;
        *reinterpret_cast<uint2*>(orow + d) =
            uint2{pack_bf16x2(oacc[qb][j][4 * g] * inv, oacc[qb][j][4 * g + 1] * inv),
                  pack_bf16x2(oacc[qb][j][4 * g + 2] * inv, oacc[qb][j][4 * g + 3] * inv)};
      }
    }
    if (a.lse && h == 0)
      a.lse[(static_cast<long long>(b) * a.T + t) * a.H + head] =
          l[qb] > 0.f ? (m[qb] + log2f(l[qb])) * 0.69314718055994531f : -INFINITY;
  }
}

// Any geometry, fp32 or bf16: one workgroup per (sequence, token, head),
// plain fp32 arithmetic, online softmax over tiles of 256 keys.
constexpr int GT = 256;
constexpr int MAX_DV_PER_T = 4;   // d_v <= 1024

__device__ __forceinline__ float pf_block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < GT / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float pf_block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < GT / 64; ++i) r += red[i];
  __syncthreads();
  return r;
}

template <typename T>
__global__ __launch_bounds__(GT) void prefill_generic_kernel(PrefillArgs a) {
  extern __shared__ float sh[];        // q[d_h + d_R] | p[GT] | red[4]
  const int DQg = a.d_h + a.d_R;
  const int D = a.d_c + a.d_R;
  float* qs = sh;
  float* ps = sh + DQg;
  float* red = ps + GT;
  const int head = blockIdx.x % a.H;
  const int t = (blockIdx.x / a.H) % a.T;
  const int b = blockIdx.x / (a.H * a.T);
  const int tid = threadIdx.x;
  const T* q = static_cast<const T*>(a.q) + ((static_cast<long long>(b) * a.T + t) * a.H + head) * DQg;
  const T* Kx = static_cast<const T*>(a.K);
  const T* Vt = static_cast<const T*>(a.Vt);
  const T* cache = static_cast<const T*>(a.cache);
  for (int k = tid; k < DQg; k += GT) qs[k] = Elem<T>::ld(q + k);
  const int nkeys = max(0, a.seq_lens[b] - a.T + t + 1);
  const float sl2 = a.scale * 1.4426950408889634f;
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[MAX_DV_PER_T];
#pragma unroll
  for (int j = 0; j < MAX_DV_PER_T; ++j) acc[j] = 0.f;
  for (int base = 0; base < nkeys; base += GT) {
    const int u = base + tid;
    float sc = -INFINITY;
    if (u < nkeys) {
      const long long sr = store_row(a, b, u);
      const T* kn = Kx + (sr * a.H + head) * a.d_h;
      const T* kr = cache + sr * D + a.d_c;
      float dot = 0.f;
      for (int k = 0; k < a.d_h; ++k) dot += qs[k] * Elem<T>::ld(kn + k);
      for (int k = 0; k < a.d_R; ++k) dot += qs[a.d_h + k] * Elem<T>::ld(kr + k);
      sc = dot * sl2;
    }
    const float bm = pf_block_max(sc, red);
    const float m_new = fmaxf(m, bm);
    const float alpha = exp2f(m - m_new);
    const float pv = (u < nkeys) ? exp2f(sc - m_new) : 0.f;
    ps[tid] = pv;
    const float bs = pf_block_sum(pv, red);   // also orders the ps writes before the reads below
    l = l * alpha + bs;
    m = m_new;
    const int nrow = min(GT, nkeys - base);
#pragma unroll
    for (int j = 0; j < MAX_DV_PER_T; ++j) {
      const int c = tid + j * GT;
      if (c < a.d_v) {
        const T* vrow = Vt + (static_cast<long long>(head) * a.d_v + c) * a.vt_ld;
        float x = acc[j] * alpha;
        for (int r = 0; r < nrow; ++r) x += ps[r] * Elem<T>::ld(vrow + vt_col(a, b, base + r));
        acc[j] = x;
      }
    }
    __syncthreads();
  }
  T* o = static_cast<T*>(a.o) + ((static_cast<long long>(b) * a.T + t) * a.H + head) * a.d_v;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int j = 0; j < MAX_DV_PER_T; ++j) {
    const int c = tid + j * GT;
    if (c < a.d_v) Elem<T>::st(o + c, acc[j] * inv);
  }
  if (a.lse && tid == 0)
    a.lse[(static_cast<long long>(b) * a.T + t) * a.H + head] =
        (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  if (a.dtype != MLA_BF16 || a.d_h != DH || a.d_R != DR || a.d_v != DV) return hipErrorInvalidValue;
  if (a.block_table && (a.block_size < 8 || (a.block_size & (a.block_size - 1)))) return hipErrorInvalidValue;
  if (a.vt_ld % 8 || a.vt_seq % 8 || (a.d_c + a.d_R) % 8) return hipErrorInvalidValue;
  constexpr int NQB = PF_NQB, NW = PF_NW, NBUF = PF_NBUF;
  constexpr int QT = NW * 32 * NQB;
  const long long blocks = static_cast<long long>(a.B) * a.H * ((a.T + QT - 1) / QT);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.block_table)
    prefill_mfma_kernel<true, NW, NQB, NBUF><<<dim3(static_cast<unsigned>(blocks)), 64 * NW, 0, stream>>>(
        a, __builtin_ctz(static_cast<unsigned>(a.block_size)));
  else
    prefill_mfma_kernel<false, NW, NQB, NBUF><<<dim3(static_cast<unsigned>(blocks)), 64 * NW, 0, stream>>>(a, 0);
  return hipGetLastError();
}

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t stream) {
  if (a.d_v > MAX_DV_PER_T * GT) return hipErrorInvalidValue;
  const size_t shmem = (static_cast<size_t>(a.d_h + a.d_R) + GT + 8) * sizeof(float);
  const long long blocks = static_cast<long long>(a.B) * a.T * a.H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.dtype == MLA_BF16)
    prefill_generic_kernel<uint16_t><<<dim3(static_cast<unsigned>(blocks)), GT, shmem, stream>>>(a);
  else
    prefill_generic_kernel<float><<<dim3(static_cast<unsigned>(blocks)), GT, shmem, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
