// Projection GEMMs and their epilogues for the query side, the output side
// and the compression of the new token.
//
// Every projection on the decode path is a skinny product: a few rows of
// activations (one per sequence) against a large weight that is read once,
// so the kernels stream the weight at HBM rate and accumulate in fp32.
//   P[split][g][m][n] = sum over the split's k range of A_g[m][k] * W_g(n, k)
// with W_g(n, k) = W[g*sWg + n*ldw + k] ([out][in] weights, "NT") or
// W[g*sWg + k*ldw + n] (the transposed use of W_UK in the absorbed query,
// "NN"). Splitting k keeps the whole chip busy when the output is small; the
// epilogues sum the splits in a fixed order (deterministic) and apply what
// the step needs next (store, rotary embedding, latent norm + cache append).
//
// bf16 path: 256 threads, a 128 (n) x 32*MT (m) output tile, 64-deep k
// steps staged through LDS (register double buffering), bf16 MFMA 32x32x16
// with fp32 accumulation. fp32 path (and shapes the MFMA path does not take):
// one thread per output element.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int GBN = 128;   // n per workgroup
constexpr int GBK = 64;    // k per step
constexpr int GTH = 256;

// LDS slot (16-byte units) of chunk kc (8 k values) of tile row r; the XOR
// keeps 16 consecutive rows of one chunk on distinct bank groups.
__device__ __forceinline__ int gslot(int r, int kc) { return r * 8 + (kc ^ ((r >> 1) & 7)); }

struct GemmP {
  const void* A; long long lda, sAg;
  const uint16_t* W; long long ldw, sWg;
  const uint16_t* W2;     // columns n >= n_split come from W2 row n - n_split (or NULL)
  int n_split;
  int M, N, K, ksplit;    // ksplit = k per split (multiple of GBK)
  float* P;
  void* out;              // direct store (streaming kernel, one split) or NULL
  long long ldo, sOg;
  int out_bf16;
};

// Activation kinds (AK): the storage dtype (A_STORE), float32 rounded once to
// bf16 (A_F32), or float32 as two bf16 terms (A_SPLIT, split_bf16x2): the
// tile then holds both terms and each k step runs two MFMAs per block.
constexpr int A_STORE = 0, A_F32_ONE = 1, A_SPLIT = 2;

template <int MT, int AK, bool W_KN>
__global__ __launch_bounds__(GTH) void gemm_mfma_kernel(GemmP p) {
  constexpr bool A_F32 = AK != A_STORE;
  constexpr int AT = AK == A_SPLIT ? 2 : 1;   // activation terms
  __shared__ __align__(16) u32x4 wt[2][GBN * 8];
  __shared__ __align__(16) u32x4 at[2][AT][32 * MT * 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * GBN;
  const int g = blockIdx.y;
  const int mblocks = (p.M + 32 * MT - 1) / (32 * MT);
  const int split = blockIdx.z / mblocks;
  const int m0 = (blockIdx.z % mblocks) * 32 * MT;
  const int k_begin = split * p.ksplit;
  const int k_end = min(p.K, k_begin + p.ksplit);
  const uint16_t* W = p.W + g * p.sWg;

  u32x4 wreg[4];
  u32x4 areg[AT][MT];

  auto load_w = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = tid & 7;
      const int n = n0 + r, k = k0 + 8 * kc;
      wreg[i] = (n < p.N && k < k_end)
                    ? *reinterpret_cast<const u32x4*>(W + static_cast<long long>(n) * p.ldw + k)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // NN weights need an 8x8 transpose; keep their staging separate for clarity.
  u32x4 wkn[8];
  auto load_w_kn = [&](int k0) {
    const int kc = tid >> 4, nc = tid & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + 8 * kc + i, n = n0 + 8 * nc;
      wkn[i] = (tid < 128 && k < k_end && n < p.N)
                   ? *reinterpret_cast<const u32x4*>(W + static_cast<long long>(k) * p.ldw + n)
                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = tid & 7;
      const int m = m0 + r, k = k0 + 8 * kc;
      if (m < p.M && k < k_end) {
        if constexpr (A_F32) {
          const float* A = static_cast<const float*>(p.A) + g * p.sAg + static_cast<long long>(m) * p.lda + k;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(A);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(A + 4);
          if constexpr (AK == A_SPLIT) {
            uint32_t hi[4], lo[4];
            split_bf16x2(x0[0], x0[1], &hi[0], &lo[0]);
            split_bf16x2(x0[2], x0[3], &hi[1], &lo[1]);
            split_bf16x2(x1[0], x1[1], &hi[2], &lo[2]);
            split_bf16x2(x1[2], x1[3], &hi[3], &lo[3]);
            areg[0][i] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            areg[AT - 1][i] = u32x4{lo[0], lo[1], lo[2], lo[3]};
          } else {
            areg[0][i] = u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                               pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
          }
        } else {
          const uint16_t* A = static_cast<const uint16_t*>(p.A) + g * p.sAg + static_cast<long long>(m) * p.lda + k;
          areg[0][i] = *reinterpret_cast<const u32x4*>(A);
        }
      } else {
#pragma unroll
        for (int t = 0; t < AT; ++t) areg[t][i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tiles = [&](int buf) {
    if constexpr (!W_KN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[buf][gslot((tid >> 3) + 32 * i, tid & 7)] = wreg[i];
    } else {
      if (tid < 128) {
        const int kc = tid >> 4, nc = tid & 15;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = __builtin_amdgcn_perm(wkn[2 * q + 1][j >> 1], wkn[2 * q][j >> 1], sel);
          wt[buf][gslot(8 * nc + j, kc)] = o;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
      for (int i = 0; i < MT; ++i) at[buf][t][gslot((tid >> 3) + 32 * i, tid & 7)] = areg[t][i];
  };

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16{};

  if (k_begin < k_end) {
    if constexpr (W_KN) load_w_kn(k_begin); else load_w(k_begin);
    load_a(k_begin);
    store_tiles(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = k_begin; k0 < k_end; k0 += GBK) {
      const bool more = k0 + GBK < k_end;
      if (more) {
        if constexpr (W_KN) load_w_kn(k0 + GBK); else load_w(k0 + GBK);
        load_a(k0 + GBK);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 av = wt[buf][gslot(32 * w + l32, 2 * j + h)];
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const u32x4 bv = at[buf][t][gslot(32 * i + l32, 2 * j + h)];
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc[i],
                                                             0, 0, 0);
          }
      }
      if (more) store_tiles(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
  // D[n][m]: lane holds m = 32i + l32, n = 32w + 8(r/4) + 4h + r%4.
  if (p.out) {
    // one split: store the product itself, out[g*sOg + m*ldo + n]
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 32 * i + l32;
      if (m >= p.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 32 * w + 8 * q + 4 * h;
        const long long o = g * p.sOg + static_cast<long long>(m) * p.ldo + n;
        if (p.out_bf16) {
          uint16_t* dst = static_cast<uint16_t*>(p.out) + o;
          if (n + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]),
                                                   pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3])};
          } else {
            for (int e = 0; e < 4 && n + e < p.N; ++e)
              dst[e] = static_cast<uint16_t>(pack_bf16x2(acc[i][4 * q + e], 0.f) & 0xffffu);
          }
        } else {
          float* dst = static_cast<float*>(p.out) + o;
          for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = acc[i][4 * q + e];
        }
      }
    }
    return;
  }
  float* P = p.P + (static_cast<long long>(split) * gridDim.y + g) * p.M * p.N;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 32 * i + l32;
    if (m >= p.M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * w + 8 * q + 4 * h;
      float* dst = P + static_cast<long long>(m) * p.N + n;
      if (n + 3 < p.N) {
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]};
      } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = acc[i][4 * q + e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming skinny GEMM for [out][in] weights ("NT"), K a multiple of 64.
//   P[split][g][m][n] = sum over the split's k range of A_g[m][k] * W_g[n][k]
// A workgroup owns 64 weight rows (output columns) and all rows of A in its
// m block (32*MT), over one k range. Weight and activation tiles of 64 k go
// HBM -> LDS by LDS-DMA (global_load_lds_dwordx4, 1 KiB per copy) through a
// ring of NS stages, so several stages of weights are in flight per
// workgroup and no register staging is needed. In LDS a 64-k row keeps its
// 16-byte chunks XOR-swizzled (chunk c of row r at slot c ^ ((r >> 1) & 7);
// fp32 activation rows: 16 chunks, slot c ^ (r & 15)); the copy picks the
// source chunk of each destination slot, and the MFMA operand reads
// (ds_read_b128, 16 lanes = 16 rows of one chunk) are bank-conflict free.
// A workgroup owns NT = 64 or 128 weight rows. Waves: w % (NT/32) picks a
// 32-column block; with NT = 64 the other bit picks a 32-k half of each
// stage, and the two k halves are summed through LDS at the end.
// ---------------------------------------------------------------------------
// weight rows per workgroup: 128 for wide outputs (halves the activation
// re-reads), 64 otherwise (more workgroups on narrow outputs)
// (very wide outputs go back to 64 so that one k split already fills the
// chip and the product is stored directly)
__host__ __device__ constexpr int stream_nt(int N) { return (N >= 4096 && N < 12288) ? 128 : 64; }
constexpr int SKT = 64;      // k per stage

template <int N>
__device__ __forceinline__ void s_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One LDS-DMA copy: each lane moves 16 bytes from its address to LDS at
// lds + 16 * lane. Inline asm so that the compiler adds no vmcnt(0) waits in
// front of later LDS reads; the kernel waits for its copies explicitly.
__device__ __forceinline__ void dma_copy(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(gptr));
}

// Wait until at most later * PW copies are in flight (later <= MAXL).
template <int PW, int MAXL>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (MAXL > 0) {
    if (later == MAXL) {
      s_wait_vmcnt<MAXL * PW>();
      return;
    }
    wait_later<PW, MAXL - 1>(later);
  } else {
    s_wait_vmcnt<0>();
  }
}

template <int NT, int MT, bool A_F32>
struct StreamCfg {
  static constexpr int NB = NT / 32;                           // 32-column blocks
  static constexpr int KH = 4 / NB;                            // k halves per stage
  static constexpr int A_ROW = A_F32 ? 256 : 128;              // bytes of one 64-k activation row
  static constexpr int W_BYTES = NT * 128;
  static constexpr int A_BYTES = 32 * MT * A_ROW;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  // one workgroup per CU with up to 144 KiB of ring, so that ~64 KiB of
  // weights are in flight per CU; never fewer than 3 stages
  static constexpr int NS0 = 144 * 1024 / STAGE;
  static constexpr int NS = NS0 > 9 ? 9 : (NS0 < 3 ? 3 : NS0);
  static constexpr int COPIES = STAGE / 1024;                  // per stage
  static constexpr int PER_WAVE = COPIES / 4;
  static_assert(COPIES % 4 == 0, "copies split evenly over four waves");
  static_assert(NS >= 3, "at least three stages");
  static_assert((NS - 1) * PER_WAVE < 64, "copies in flight fit the vmcnt counter");
};

template <int NT, int MT, int AK>
__global__ __launch_bounds__(GTH) void gemm_stream_kernel(GemmP p) {
  constexpr bool A_F32 = AK != A_STORE;
  using C = StreamCfg<NT, MT, A_F32>;
  __shared__ __align__(1024) char smem[C::NS * C::STAGE];
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)smem));
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5, l32 = lane & 31;
  const int nh = w % C::NB, kh = w / C::NB;
  const int n0 = blockIdx.x * NT;
  const int g = blockIdx.y;
  const int mblocks = (p.M + 32 * MT - 1) / (32 * MT);
  const int split = blockIdx.z / mblocks;
  const int m0 = (blockIdx.z % mblocks) * 32 * MT;
  const int k_begin = split * p.ksplit;
  const int k_end = min(p.K, k_begin + p.ksplit);
  const int nsteps = k_end > k_begin ? (k_end - k_begin) / SKT : 0;
  // a tile lies wholly on one side of n_split (a multiple of NT)
  const bool second = p.W2 != nullptr && n0 >= p.n_split;
  const uint16_t* W = second ? p.W2 : p.W + g * p.sWg;
  const int wrow0 = second ? p.n_split : 0;

  // copy i of a stage (0..COPIES-1) for this lane: source address and LDS offset
  auto issue_stage = [&](int t) {
    const int kb = k_begin + t * SKT;
    const uint32_t st = sbase + (t % C::NS) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::PER_WAVE; ++j) {
      const int i = w * C::PER_WAVE + j;
      if (i < NT / 8) {                              // weight rows 8i..8i+7
        const int r = 8 * i + (lane >> 3), slot = lane & 7;
        const int c = slot ^ ((r >> 1) & 7);
        const int n = min(n0 + r, p.N - 1) - wrow0;
        dma_copy(W + static_cast<long long>(n) * p.ldw + kb + 8 * c, st + 1024 * i);
      } else if constexpr (!A_F32) {                  // activation rows, bf16
        const int a = i - NT / 8;
        const int r = 8 * a + (lane >> 3), slot = lane & 7;
        const int c = slot ^ ((r >> 1) & 7);
        const int m = min(m0 + r, p.M - 1);
        const uint16_t* A = static_cast<const uint16_t*>(p.A) + g * p.sAg;
        dma_copy(A + static_cast<long long>(m) * p.lda + kb + 8 * c, st + C::W_BYTES + 1024 * a);
      } else {                                        // activation rows, fp32
        const int a = i - NT / 8;
        const int r = 4 * a + (lane >> 4), slot = lane & 15;
        const int c = slot ^ (r & 15);
        const int m = min(m0 + r, p.M - 1);
        const float* A = static_cast<const float*>(p.A) + g * p.sAg;
        dma_copy(A + static_cast<long long>(m) * p.lda + kb + 4 * c, st + C::W_BYTES + 1024 * a);
      }
    }
  };

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16{};

  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < C::NS - 1; ++j)
      if (j < nsteps) issue_stage(j);
    for (int t = 0; t < nsteps; ++t) {
      // stage t landed: only the copies of stages t+1 .. t+NS-2 may still fly
      const int later = min(nsteps - 1 - t, C::NS - 2);
      wait_later<C::PER_WAVE, C::NS - 2>(later);
      // plain barrier: __syncthreads would also wait for the copies in flight
      asm volatile("s_barrier" ::: "memory");
      // every wave is past stage t-1: its slot takes stage t+NS-1
      if (t + C::NS - 1 < nsteps) issue_stage(t + C::NS - 1);
      const char* st = smem + (t % C::NS) * C::STAGE;
#pragma unroll
      for (int j2 = 0; j2 < 4 / C::KH; ++j2) {
        const int j = (4 / C::KH) * kh + j2;          // k16 step of this wave
        const int rw = 32 * nh + l32, cw = 2 * j + h;
        const u32x4 wv = *reinterpret_cast<const u32x4*>(st + 16 * (rw * 8 + (cw ^ ((rw >> 1) & 7))));
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int ra = 32 * i + l32;
          bf16x8 av;
          if constexpr (!A_F32) {
            av = *reinterpret_cast<const bf16x8*>(st + C::W_BYTES + 16 * (ra * 8 + (cw ^ ((ra >> 1) & 7))));
          } else {
            const char* arow = st + C::W_BYTES + ra * 256;
            const int c0 = 2 * cw, c1 = 2 * cw + 1;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(arow + 16 * (c0 ^ (ra & 15)));
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(arow + 16 * (c1 ^ (ra & 15)));
            if constexpr (AK == A_F32_ONE) {
              av = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                                    pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])});
            } else {
              // two bf16 terms (split_bf16x2), two MFMAs
              uint32_t hi[4], lo[4];
              split_bf16x2(x0[0], x0[1], &hi[0], &lo[0]);
              split_bf16x2(x0[2], x0[3], &hi[1], &lo[1]);
              split_bf16x2(x1[0], x1[1], &hi[2], &lo[2]);
              split_bf16x2(x1[2], x1[3], &hi[3], &lo[3]);
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]}),
                  acc[i], 0, 0, 0);
              av = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
            }
          }
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv), av, acc[i], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (C::KH == 2) {
    // sum the two k halves: waves 2,3 hand their accumulators to waves 0,1
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((nh * MT + i) * 16 + r) * 64 + lane] = acc[i][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] += red[((nh * MT + i) * 16 + r) * 64 + lane];
  }
  // D[n][m]: lane holds m = 32i + l32, n = 32nh + 8(r/4) + 4h + r%4.
  if (p.out) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 32 * i + l32;
      if (m >= p.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 32 * nh + 8 * q + 4 * h;
        const long long o = g * p.sOg + static_cast<long long>(m) * p.ldo + n;
        if (p.out_bf16) {
          uint16_t* dst = static_cast<uint16_t*>(p.out) + o;
          if (n + 3 < p.N && (o & 3) == 0) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]),
                                                        pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3]));
          } else {
            for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = f32_to_bf16(acc[i][4 * q + e]);
          }
        } else {
          float* dst = static_cast<float*>(p.out) + o;
          for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = acc[i][4 * q + e];
        }
      }
    }
    return;
  }
  float* P = p.P + (static_cast<long long>(split) * gridDim.y + g) * p.M * p.N;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 32 * i + l32;
    if (m >= p.M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * nh + 8 * q + 4 * h;
      float* dst = P + static_cast<long long>(m) * p.N + n;
      if (n + 3 < p.N) {
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]};
      } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = acc[i][4 * q + e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tall products (many rows of activations, e.g. expanding every cached
// latent row into per-head keys or values): bf16 A [M][K] (lda) times bf16
// W [N][K] (ldw), stored directly as bf16 out[g*sOg + m*ldo + n]; K a
// multiple of 64, one k range. A workgroup owns a 128 (n) x 128 (m) tile;
// its four waves own 64 x 64 each (2 x 2 MFMA 32x32x16 blocks, four operand
// reads per four MFMAs). Stages of 64 k (16 KiB of weights, 16 KiB of
// activations) go HBM -> LDS by LDS-DMA, double buffered, with the same
// swizzle as the streaming kernel; 64 KiB of LDS lets two workgroups share
// a CU, so one's prologue and stores overlap the other's MFMAs. The
// epilogue stages the tile in LDS as rows of 128 outputs and stores each row
// as one contiguous 256-byte run.
// ---------------------------------------------------------------------------
constexpr int TT_N = 128, TT_M = 128;
constexpr int TT_WB = TT_N * 128, TT_AB = TT_M * 128;     // bytes per stage
constexpr int TT_STAGE = TT_WB + TT_AB;                   // 32 KiB
constexpr int TT_NS = 2;
constexpr int TT_PW = TT_STAGE / 1024 / 4;                 // copies per wave per stage: 8
constexpr int TT_OROW = TT_N * 2 + 16;                    // staged output row stride (bytes)
static_assert(TT_M * TT_OROW <= TT_NS * TT_STAGE, "output tile fits in the ring");

__global__ __launch_bounds__(256) void gemm_tall_kernel(const uint16_t* __restrict__ A, long long lda,
                                                        long long sAg, const uint16_t* __restrict__ W,
                                                        long long ldw, long long sWg, uint16_t* __restrict__ out,
                                                        long long ldo, long long sOg, int M, int N, int K) {
  __shared__ __align__(1024) char smem[TT_NS * TT_STAGE];
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)smem));
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5, l32 = lane & 31;
  const int wn = w & 1, wm = w >> 1;
  const int n0 = blockIdx.x * TT_N, m0 = blockIdx.y * TT_M, g = blockIdx.z;
  const uint16_t* Wg = W + g * sWg;
  const uint16_t* Ag = A + g * sAg;
  const int nsteps = K / 64;

  auto issue_stage = [&](int t) {
    const int kb = t * 64;
    const uint32_t st = sbase + (t % TT_NS) * TT_STAGE;
#pragma unroll
    for (int j = 0; j < TT_PW; ++j) {
      const int i = w * TT_PW + j;                   // copy 0..47
      const int r8 = lane >> 3, c = (lane & 7);
      if (i < TT_N / 8) {                            // weight rows 8i..8i+7
        const int r = 8 * i + r8;
        const int n = min(n0 + r, N - 1);
        dma_copy(Wg + static_cast<long long>(n) * ldw + kb + 8 * (c ^ ((r >> 1) & 7)), st + 1024 * i);
      } else {                                       // activation rows
        const int a = i - TT_N / 8, r = 8 * a + r8;
        const int m = min(m0 + r, M - 1);
        dma_copy(Ag + static_cast<long long>(m) * lda + kb + 8 * (c ^ ((r >> 1) & 7)), st + TT_WB + 1024 * a);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

#pragma unroll
  for (int t = 0; t < TT_NS - 1; ++t)
    if (t < nsteps) issue_stage(t);
  for (int t = 0; t < nsteps; ++t) {
    wait_later<TT_PW, TT_NS - 2>(min(nsteps - 1 - t, TT_NS - 2));
    asm volatile("s_barrier" ::: "memory");
    if (t + TT_NS - 1 < nsteps) issue_stage(t + TT_NS - 1);
    const char* st = smem + (t % TT_NS) * TT_STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {                    // k16 steps of the stage
      const int cw = 2 * j + h;
      u32x4 wv[2], av[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int rw = 64 * wn + 32 * nb + l32;
        wv[nb] = *reinterpret_cast<const u32x4*>(st + 16 * (rw * 8 + (cw ^ ((rw >> 1) & 7))));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int ra = 64 * wm + 32 * mb + l32;
        av[mb] = *reinterpret_cast<const u32x4*>(st + TT_WB + 16 * (ra * 8 + (cw ^ ((ra >> 1) & 7))));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv[nb]),
                                                                __builtin_bit_cast(bf16x8, av[mb]), acc[nb][mb],
                                                                0, 0, 0);
    }
  }
  // D[n][m] of block (nb, mb): lane holds m = 32mb + l32, n = 32nb + 8(r/4) + 4h + r%4
  // (within the wave's 128 x 64). Stage as rows m of 256 outputs, then store rows.
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int ml = 64 * wm + 32 * mb + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 64 * wn + 32 * nb + 8 * q + 4 * h;
        *reinterpret_cast<uint2*>(smem + ml * TT_OROW + 2 * nl) =
            make_uint2(pack_bf16x2(acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1]),
                       pack_bf16x2(acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]));
      }
    }
  __syncthreads();
  uint16_t* og = out + g * sOg;
  for (int idx = tid; idx < TT_M * (TT_N / 8); idx += 256) {
    const int row = idx / (TT_N / 8), piece = idx % (TT_N / 8);
    const int m = m0 + row, n = n0 + 8 * piece;
    if (m >= M || n >= N) continue;
    const char* src = smem + row * TT_OROW + 16 * piece;
    uint16_t* dst = og + static_cast<long long>(m) * ldo + n;
    if (n + 8 <= N && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = reinterpret_cast<const uint16_t*>(src)[e];
    }
  }
}

// One thread per output element (fp32 storage, or shapes the MFMA kernel
// does not take). Same partial layout as the MFMA kernel.
template <typename TA, typename TW>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const TA* __restrict__ A, long long lda,
                                                         long long sAg, const TW* __restrict__ W,
                                                         long long ldw, long long sWg, int w_kn,
                                                         int M, int N, int K, int G, int ksplit,
                                                         float* __restrict__ P) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  const int g = blockIdx.z % G;
  const int split = blockIdx.z / G;
  if (n >= N) return;
  const int k0 = split * ksplit, k1 = min(K, k0 + ksplit);
  const TA* a = A + g * sAg + static_cast<long long>(m) * lda;
  const TW* wp = W + g * sWg;
  float acc = 0.f;
  if (!w_kn) {
    const TW* wr = wp + static_cast<long long>(n) * ldw;
    for (int k = k0; k < k1; ++k) acc += Elem<TA>::ld(a + k) * Elem<TW>::ld(wr + k);
  } else {
    for (int k = k0; k < k1; ++k) acc += Elem<TA>::ld(a + k) * Elem<TW>::ld(wp + static_cast<long long>(k) * ldw + n);
  }
  P[((static_cast<long long>(split) * G + g) * M + m) * N + n] = acc;
}

template <typename TO>
__global__ void reduce_store_kernel(const float* __restrict__ P, int splits, int G, int M, int N,
                                    TO* __restrict__ out, long long ldo, long long sOg) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  const long long total = static_cast<long long>(G) * M * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  const int m = static_cast<int>((idx / N) % M);
  const int g = static_cast<int>(idx / (static_cast<long long>(N) * M));
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += P[s * total + idx];
  Elem<TO>::st(out + g * sOg + m * ldo + n, v);
}

// The same sum (G = 1) stored twice: in float32, and rounded once to bf16 for
// the products that take the activation rounded (the rounding the streaming
// GEMM applies to a float32 activation on load, so their results are the same).
__global__ void reduce_store_dual_kernel(const float* __restrict__ P, int splits, int M, int N,
                                         float* __restrict__ out32, uint16_t* __restrict__ out16) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  const long long total = static_cast<long long>(M) * N;
  if (idx >= total) return;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += P[s * total + idx];
  out32[idx] = v;
  out16[idx] = f32_to_bf16(v);
}

// A value stored as two terms of the storage type: the nearest value, then
// the nearest value of the remainder (zero for float32).
template <typename TO> struct TwoTerm;
template <> struct TwoTerm<float> {
  __device__ static __forceinline__ void st(float* hi, float* lo, float v) { *hi = v; *lo = 0.f; }
};
template <> struct TwoTerm<uint16_t> {
  __device__ static __forceinline__ void st(uint16_t* hi, uint16_t* lo, float v) {
    const uint16_t h = f32_to_bf16(v);
    *hi = h;
    *lo = f32_to_bf16(v - bf16_to_f32(h));
  }
};

// Rotary projection [M][G*d_R] -> rotated, stored at out[m*ldo + g*sOg + j]
// and, as its second term, at out[m*ldo + g*sOg + d_R + j].
template <typename TO>
__global__ __launch_bounds__(256) void reduce_rope_kernel(const float* __restrict__ P, int splits, int M, int G,
                                                          int d_R, const int32_t* __restrict__ pos, float theta,
                                                          TO* __restrict__ out, long long ldo, long long sOg) {
  // Workgroup (chunk x, row m): pairs 256x .. 256x + 255 of row m, one per
  // thread, all split loads of a thread in flight together. The angle of
  // pair j depends on (m, j) only: the workgroup evaluates each angle it
  // needs once and every head in the chunk reuses it.
  __shared__ float cs[2 * 512];
  const int half = d_R / 2;
  const int row_pairs = G * half;
  const long long total = static_cast<long long>(M) * G * d_R;
  const int p0 = blockIdx.x * 256;
  const int nj = min(half, 256);
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    for (int t = threadIdx.x; t < nj; t += 256) {
      const int j = (half <= 256) ? t : (p0 + t) % half;
      rope_cs(pos[m], j, d_R, theta, &cs[2 * t], &cs[2 * t + 1]);
    }
    __syncthreads();
    const int pi = p0 + threadIdx.x;
    if (pi < row_pairs) {
      const int g = pi / half, j = pi % half;
      const int jt = (half <= 256) ? j : pi - p0;
      const long long e0 = static_cast<long long>(m) * G * d_R + 2LL * pi;
      float x0 = 0.f, x1 = 0.f;
      int s = 0;
      for (; s + 4 <= splits; s += 4) {
        const float2 v0 = *reinterpret_cast<const float2*>(P + s * total + e0);
        const float2 v1 = *reinterpret_cast<const float2*>(P + (s + 1) * total + e0);
        const float2 v2 = *reinterpret_cast<const float2*>(P + (s + 2) * total + e0);
        const float2 v3 = *reinterpret_cast<const float2*>(P + (s + 3) * total + e0);
        x0 += v0.x + v1.x + v2.x + v3.x;
        x1 += v0.y + v1.y + v2.y + v3.y;
      }
      for (; s < splits; ++s) {
        const float2 v = *reinterpret_cast<const float2*>(P + s * total + e0);
        x0 += v.x;
        x1 += v.y;
      }
      const float c = cs[2 * jt], sn = cs[2 * jt + 1];
      TO* o = out + static_cast<long long>(m) * ldo + g * sOg + 2 * j;
      TwoTerm<TO>::st(o, o + d_R, x0 * c - x1 * sn);
      TwoTerm<TO>::st(o + 1, o + d_R + 1, x0 * sn + x1 * c);
    }
    __syncthreads();   // the angles of the next row overwrite cs
  }
}

// One workgroup per sequence, one thread per column of the row (up to 1024):
// sum the splits of [c ; k_R], optionally RMS-normalise c ("Understanding
// MLA" (Dong), A2: norm on the latent only), rotate k_R at the token's
// position, round and write the cache row. Every thread issues the loads of
// all its splits at once, so the sums cost about one memory round trip.
template <typename T>
__global__ __launch_bounds__(1024) void append_kernel(const float* __restrict__ Pc, int splits_c, int ldc,
                                                      const float* __restrict__ Pr, int splits_r, int ldr, int M,
                                                      int d_c, int d_R, const T* __restrict__ gamma,
                                                      float eps, const int32_t* __restrict__ pos,
                                                      float theta, mla_cache cache) {
  extern __shared__ float row[];    // d_c + d_R floats, then 16 for the reduction
  const int m = blockIdx.x;
  const int D = d_c + d_R;
  float* red = row + D;
  float ss = 0.f;
  // Split sums: four independent chains; fixed order, hence deterministic.
  auto split_sum = [&](const float* P, int splits, int ld, int c) {
    float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
    const long long stride = static_cast<long long>(M) * ld;
    const float* q = P + static_cast<long long>(m) * ld + c;
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
      v0 += q[s * stride];
      v1 += q[(s + 1) * stride];
      v2 += q[(s + 2) * stride];
      v3 += q[(s + 3) * stride];
    }
    for (; s < splits; ++s) v0 += q[s * stride];
    return (v0 + v1) + (v2 + v3);
  };
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const float v = c < d_c ? split_sum(Pc, splits_c, ldc, c) : split_sum(Pr, splits_r, ldr, c - d_c);
    row[c] = v;
    if (c < d_c) ss += v * v;
  }
  float rinv = 1.f;
  if (gamma) {
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  if (gamma) {
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red[i];
    rinv = rsqrtf(tot / d_c + eps);
  }
  const int t = pos[m];
  T* dst;
  if (cache.block_table == nullptr) {
    dst = static_cast<T*>(cache.data) + (static_cast<long long>(m) * cache.capacity + t) * D;
  } else {
    const int blk = cache.block_table[m * cache.max_blocks + t / cache.block_size];
    dst = static_cast<T*>(cache.data) +
          (static_cast<long long>(blk) * cache.block_size + t % cache.block_size) * D;
  }
  for (int c = threadIdx.x; c < d_c + d_R / 2; c += blockDim.x) {
    if (c < d_c) {
      float v = row[c];
      if (gamma) v = v * rinv * Elem<T>::ld(gamma + c);
      Elem<T>::st(dst + c, v);
    } else {
      const int j = c - d_c;
      float cs, sn;
      rope_cs(t, j, d_R, theta, &cs, &sn);
      const float x0 = row[d_c + 2 * j], x1 = row[d_c + 2 * j + 1];
      Elem<T>::st(dst + d_c + 2 * j, x0 * cs - x1 * sn);
      Elem<T>::st(dst + d_c + 2 * j + 1, x0 * sn + x1 * cs);
    }
  }
}

// Offline weight composition, C(g, m, n) = sum_k X(g, k, m) Y(g, k, n), with
// element strides X(g, k, m) = X[g*xg + k*xk + m*xm], Y(g, k, n) =
// Y[g*yg + k*yk + n], C(g, m, n) = C[g*cg + m*cm + n]; fp32 accumulation,
// one thread per output element, the X value shared by the workgroup.
template <typename T>
__global__ __launch_bounds__(256) void compose_kernel(const T* __restrict__ X, long long xg, long long xk,
                                                      long long xm, const T* __restrict__ Y, long long yg,
                                                      long long yk, T* __restrict__ C, long long cg, long long cm,
                                                      int N, int K) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  const int g = blockIdx.z;
  if (n >= N) return;
  const T* x = X + g * xg + m * xm;
  const T* y = Y + g * yg + n;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += Elem<T>::ld(x + k * xk) * Elem<T>::ld(y + k * yk);
  Elem<T>::st(C + g * cg + m * cm + n, acc);
}

bool mfma_ok(const GemmArgs& a) {
  if (a.dtype != MLA_BF16) return false;
  if (a.K % 8 || a.lda % 8 || a.ldw % 8 || a.sAg % 8 || a.sWg % 8) return false;
  if (a.w_kn && a.N % 8) return false;
  if ((reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.W)) & 15) return false;
  return true;
}

// The streaming kernel is for skinny products (every workgroup re-streams its
// activation rows for each column tile); taller products take the tiled kernel.
bool stream_ok(const GemmArgs& a) { return mfma_ok(a) && !a.w_kn && a.K % SKT == 0 && a.M <= 128; }

int device_cus() {
  static thread_local int dev_cached = -1, cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cus;
  if (dev != dev_cached) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    dev_cached = dev;
  }
  return cus;
}

}  // namespace

int gemm_splits(int M, int N, int K, int G, int dtype) {
  (void)dtype;
  const int ksteps = (K + GBK - 1) / GBK;
  const int mblocks = (M + 127) / 128;
  const int nt = stream_nt(N);
  const long long tiles = static_cast<long long>((N + nt - 1) / nt) * G * mblocks;
  const long long target = 256;   // about one workgroup per compute unit
  long long s = target / tiles;   // whole rounds: never spill into a partial second round
  // Each split writes an fp32 partial of M x N that the epilogue reads back
  // shortly after (mostly from the last-level cache); keep that traffic
  // (8*S*M*N bytes) within the weight bytes (2*N*K), i.e. S <= K / (4 M).
  const long long s_traffic = K / (4LL * (M > 0 ? M : 1));
  if (s > s_traffic) s = s_traffic;
  if (s > ksteps) s = ksteps;
  if (s < 1) s = 1;
  // k per split is a whole number of steps; recompute the count that covers K
  const int kper = static_cast<int>((ksteps + s - 1) / s) * GBK;
  return (K + kper - 1) / kper;
}

bool gemm_direct(const GemmArgs& a) { return a.out != nullptr && a.splits == 1 && mfma_ok(a); }

bool gemm_concat_ok(const GemmArgs& a) {
  return stream_ok(a) && a.G == 1 && a.n_split > 0 && a.n_split % stream_nt(a.N) == 0 &&
         (reinterpret_cast<uintptr_t>(a.W2) & 15) == 0;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.W2 && !gemm_concat_ok(a)) return hipErrorInvalidValue;
  // m blocks (of up to 128 rows) times k splits share the z grid dimension
  if (static_cast<long long>(a.splits) * ((a.M + 127) / 128) > 65535) return hipErrorInvalidValue;
  const int splits = a.splits;
  const int ak = a.a_f32 ? (a.a_split ? A_SPLIT : A_F32_ONE) : A_STORE;
  const int ksteps = (a.K + GBK - 1) / GBK;
  const int kper = ((ksteps + splits - 1) / splits) * GBK;
  if (stream_ok(a)) {
    GemmP p{a.A, a.lda, a.sAg, static_cast<const uint16_t*>(a.W), a.ldw, a.sWg,
            static_cast<const uint16_t*>(a.W2), a.n_split, a.M, a.N, a.K, kper, a.P, nullptr, 0, 0, 0};
    if (gemm_direct(a)) {
      p.out = a.out;
      p.ldo = a.ldo;
      p.sOg = a.sOg;
      p.out_bf16 = a.out_dtype == MLA_BF16;
    }
    const int MT = a.M <= 32 ? 1 : a.M <= 64 ? 2 : 4;
    const int nt = stream_nt(a.N);
    const int mblocks = (a.M + 32 * MT - 1) / (32 * MT);
    const dim3 grid((a.N + nt - 1) / nt, a.G, splits * mblocks);
#define MLA_STREAM(NTV, MTV)                                                                     \
  if (ak == A_SPLIT) gemm_stream_kernel<NTV, MTV, A_SPLIT><<<grid, GTH, 0, stream>>>(p);         \
  else if (ak == A_F32_ONE) gemm_stream_kernel<NTV, MTV, A_F32_ONE><<<grid, GTH, 0, stream>>>(p); \
  else gemm_stream_kernel<NTV, MTV, A_STORE><<<grid, GTH, 0, stream>>>(p);
    if (nt == 128) {
      if (MT == 1) { MLA_STREAM(128, 1) } else if (MT == 2) { MLA_STREAM(128, 2) } else { MLA_STREAM(128, 4) }
    } else {
      if (MT == 1) { MLA_STREAM(64, 1) } else if (MT == 2) { MLA_STREAM(64, 2) } else { MLA_STREAM(64, 4) }
    }
#undef MLA_STREAM
    return hipGetLastError();
  }
  if (mfma_ok(a)) {
    GemmP p{a.A, a.lda, a.sAg, static_cast<const uint16_t*>(a.W), a.ldw, a.sWg,
            static_cast<const uint16_t*>(a.W2), a.n_split, a.M, a.N, a.K, kper, a.P, nullptr, 0, 0, 0};
    if (gemm_direct(a)) {
      p.out = a.out;
      p.ldo = a.ldo;
      p.sOg = a.sOg;
      p.out_bf16 = a.out_dtype == MLA_BF16;
    }
    const int MT = a.M <= 32 ? 1 : a.M <= 64 ? 2 : 4;
    const int mblocks = (a.M + 32 * MT - 1) / (32 * MT);
    const dim3 grid((a.N + GBN - 1) / GBN, a.G, splits * mblocks);
#define MLA_GEMM_AK(MTV, AKV)                                                                    \
  if (a.w_kn) gemm_mfma_kernel<MTV, AKV, true><<<grid, GTH, 0, stream>>>(p);                     \
  else gemm_mfma_kernel<MTV, AKV, false><<<grid, GTH, 0, stream>>>(p);
#define MLA_GEMM(MTV)                                                                            \
  if (ak == A_SPLIT) { MLA_GEMM_AK(MTV, A_SPLIT) }                                               \
  else if (ak == A_F32_ONE) { MLA_GEMM_AK(MTV, A_F32_ONE) }                                      \
  else { MLA_GEMM_AK(MTV, A_STORE) }
    if (MT == 1) { MLA_GEMM(1) } else if (MT == 2) { MLA_GEMM(2) } else { MLA_GEMM(4) }
#undef MLA_GEMM
#undef MLA_GEMM_AK
    return hipGetLastError();
  }
  const dim3 grid((a.N + 255) / 256, a.M, a.G * splits);
  if (a.dtype == MLA_BF16) {
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    if (a.a_f32)
      gemm_simt_kernel<float, uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const float*>(a.A), a.lda, a.sAg, W, a.ldw, a.sWg, a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
    else
      gemm_simt_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const uint16_t*>(a.A), a.lda, a.sAg, W, a.ldw, a.sWg, a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
  } else {
    gemm_simt_kernel<float, float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(a.A), a.lda, a.sAg, static_cast<const float*>(a.W), a.ldw, a.sWg,
        a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
  }
  return hipGetLastError();
}

bool gemm_tall_ok(const GemmArgs& a) {
  return a.dtype == MLA_BF16 && !a.a_f32 && !a.w_kn && !a.W2 && a.out && a.out_dtype == MLA_BF16 && a.K % 64 == 0 &&
         a.M > 128 && a.lda % 8 == 0 && a.ldw % 8 == 0 && a.sAg % 8 == 0 && a.sWg % 8 == 0 &&
         ((reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.W)) & 15) == 0 &&
         (a.M + TT_M - 1) / TT_M <= 65535 && a.G <= 65535;
}

hipError_t launch_gemm_tall(const GemmArgs& a, hipStream_t stream) {
  if (!gemm_tall_ok(a)) return hipErrorInvalidValue;
  const dim3 grid((a.N + TT_N - 1) / TT_N, (a.M + TT_M - 1) / TT_M, a.G);
  gemm_tall_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(a.A), a.lda, a.sAg,
                                             static_cast<const uint16_t*>(a.W), a.ldw, a.sWg,
                                             static_cast<uint16_t*>(a.out), a.ldo, a.sOg, a.M, a.N, a.K);
  return hipGetLastError();
}

hipError_t launch_reduce_store(const float* P, int splits, int G, int M, int N, void* out,
                               long long ldo, long long sOg, int out_dtype, hipStream_t stream) {
  const long long total = static_cast<long long>(G) * M * N;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (out_dtype == MLA_BF16)
    reduce_store_kernel<uint16_t><<<grid, 256, 0, stream>>>(P, splits, G, M, N, static_cast<uint16_t*>(out), ldo, sOg);
  else
    reduce_store_kernel<float><<<grid, 256, 0, stream>>>(P, splits, G, M, N, static_cast<float*>(out), ldo, sOg);
  return hipGetLastError();
}

hipError_t launch_reduce_store_dual(const float* P, int splits, int M, int N, float* out32, uint16_t* out16,
                                    hipStream_t stream) {
  const long long total = static_cast<long long>(M) * N;
  reduce_store_dual_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(P, splits, M, N,
                                                                                              out32, out16);
  return hipGetLastError();
}

hipError_t launch_reduce_rope(const float* P, int splits, int M, int G, int d_R, const int32_t* pos,
                              float theta, void* out, long long ldo, long long sOg, int out_dtype,
                              hipStream_t stream) {
  if (d_R > 1024 || d_R % 2) return hipErrorInvalidValue;
  const long long row_pairs = static_cast<long long>(G) * (d_R / 2);
  const dim3 grid(static_cast<unsigned>((row_pairs + 255) / 256), static_cast<unsigned>(M < 65535 ? M : 65535));
  if (out_dtype == MLA_BF16)
    reduce_rope_kernel<uint16_t><<<grid, 256, 0, stream>>>(P, splits, M, G, d_R, pos, theta, static_cast<uint16_t*>(out), ldo, sOg);
  else
    reduce_rope_kernel<float><<<grid, 256, 0, stream>>>(P, splits, M, G, d_R, pos, theta, static_cast<float*>(out), ldo, sOg);
  return hipGetLastError();
}

// Rotary query of the prefill entries into the absorbed query rows: rows of
// src [n][...] hold q_R at src + k*lds + off_src; dst rows get it at
// dst + k*ldd + off_dst followed by a zero second term (the given q_R is
// exact in the storage type).
template <typename T>
__global__ __launch_bounds__(256) void rope_query_copy_kernel(const T* __restrict__ src, long long lds, int off_src,
                                                              T* __restrict__ dst, long long ldd, int off_dst,
                                                              int d_R, long long n) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  if (idx >= n * d_R) return;
  const long long k = idx / d_R;
  const int j = static_cast<int>(idx % d_R);
  T* o = dst + k * ldd + off_dst + j;
  o[0] = src[k * lds + off_src + j];
  o[d_R] = T(0);
}

hipError_t launch_rope_query_copy(const void* src, long long lds, int off_src, void* dst, long long ldd, int off_dst,
                                  int d_R, long long n, int dtype, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n * d_R + 255) / 256));
  if (dtype == MLA_BF16)
    rope_query_copy_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(src), lds, off_src,
                                                                static_cast<uint16_t*>(dst), ldd, off_dst, d_R, n);
  else
    rope_query_copy_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(src), lds, off_src,
                                                             static_cast<float*>(dst), ldd, off_dst, d_R, n);
  return hipGetLastError();
}

hipError_t launch_append(const float* Pc, int splits_c, int ldc, const float* Pr, int splits_r, int ldr, int M,
                         int d_c, int d_R,
                         const void* gamma, float eps, const int32_t* pos, float theta,
                         const mla_cache& cache, int dtype, hipStream_t stream) {
  const size_t shmem = (static_cast<size_t>(d_c + d_R) + 16) * sizeof(float);
  const int threads = std::min(1024, (d_c + d_R + 63) / 64 * 64);
  if (dtype == MLA_BF16)
    append_kernel<uint16_t><<<M, threads, shmem, stream>>>(Pc, splits_c, ldc, Pr, splits_r, ldr, M, d_c, d_R,
                                                           static_cast<const uint16_t*>(gamma), eps, pos, theta,
                                                           cache);
  else
    append_kernel<float><<<M, threads, shmem, stream>>>(Pc, splits_c, ldc, Pr, splits_r, ldr, M, d_c, d_R,
                                                        static_cast<const float*>(gamma), eps, pos, theta, cache);
  return hipGetLastError();
}


hipError_t launch_compose(const void* X, long long xg, long long xk, long long xm, const void* Y, long long yg,
                          long long yk, void* C, long long cg, long long cm, int G, int M, int N, int K, int dtype,
                          hipStream_t stream) {
  const dim3 grid((N + 255) / 256, M, G);
  if (dtype == MLA_BF16)
    compose_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(X), xg, xk, xm,
                                                       static_cast<const uint16_t*>(Y), yg, yk,
                                                       static_cast<uint16_t*>(C), cg, cm, N, K);
  else
    compose_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(X), xg, xk, xm,
                                                    static_cast<const float*>(Y), yg, yk, static_cast<float*>(C),
                                                    cg, cm, N, K);
  return hipGetLastError();
}

}  // namespace mla
