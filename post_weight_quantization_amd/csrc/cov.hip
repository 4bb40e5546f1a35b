// Stage 1: covariances H_X = Xq^T Xq, D = dX^T Xq, H_G = G^T G (scaled by alpha).
//
// KronQ summary (hyper.ai), Method: the Fisher of a linear layer factors under
// K-FAC as H ~ H_X (x) H_G with H_X = E[x x^T] and H_G = E[g g^T]; the GPTAQ
// objective adds the drift term dX X^T. With token-major inputs (one token
// per row), each output is a "TN" product C[i][j] = sum_t A[t][i] B[t][j].
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * a drift pre-pass writes dX = bf16_rne(X - Xq) once (packed fp32 -> bf16
//     conversion, nearest even);
//   * work items are 256 x 256 output tiles over a token range; H_X and H_G
//     take lower-triangle tiles only, D all tiles; one launch covers all three;
//   * a workgroup (4 waves of 128 x 128, 256 accumulator registers per lane)
//     streams stages of 32 tokens x 256 channels per operand from HBM straight
//     into LDS with global_load_lds_dwordx4 through a 4-deep ring, and reads
//     MFMA operands with transposing LDS reads (ds_read_b64_tr_b16) from an
//     XOR-swizzled layout (16-byte chunk c of token row r at c ^ 4(r & 3));
//   * the host builds the schedule: tiles are enumerated in bands of 8 tile
//     rows so that 32 consecutive tiles form an 8 x 4 block touching 12
//     channel strips; each group of 32 tiles and token split fills the 32
//     CUs of one XCD for one round (workgroup b runs on XCD b % 8), so those
//     workgroups stream the same tokens of few strips through one L2; the
//     items left for a last, partial round are cut into shorter token pieces
//     spread over all XCDs so no CU idles while a few finish;
//   * an item that covers all tokens of its tile applies alpha/beta and
//     mirrors lower tiles of H_X and H_G itself; otherwise it writes its
//     partial tile to a slot of a pool and a reduction kernel sums each
//     tile's slots in a fixed order (deterministic), then does the same.
// fp32 path (small workloads): the generic fp32 MFMA GEMM with transposed A.
#include <vector>

#include "kq_internal.h"

namespace kq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int CT = 256;            // output tile edge (channels)
constexpr int KS = 32;             // tokens per LDS stage
constexpr int NST = 4;             // LDS ring depth (stages)
constexpr int ROWB = CT * 2;       // bytes per token row of a raw tile
constexpr int STB = KS * ROWB;     // bytes per operand stage (16 KB)

enum Kind { K_HX = 0, K_D = 1, K_HG = 2 };
enum Mode { M_DIAG = 0, M_PAIR = 1 };

// One work item: tile (I, J) of matrix `kind` over tokens [t0, t1). slot < 0:
// write the output tile directly; else write the partial to pool slot `slot`.
struct CovItem {
  int32_t kind, I, J, slot;
  int64_t t0, t1;
};

// A tile whose partials sit in pool slots slot0 .. slot0 + count - 1.
struct CovRed {
  int32_t kind, I, J, count;
  int64_t slot0;
};

struct CovArgs {
  const uint16_t* Xq;
  const uint16_t* dX;  // bf16 drift, token-major (written by the drift pre-pass)
  const uint16_t* G;
  int64_t d_in, d_out;
  float alpha, beta;
  float* out[3];       // H_X, D, H_G
  const CovItem* items;
  float* pool;         // partial tiles, 256 x 256 floats per slot
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Raw tiles keep the global layout (token rows of 256 channels); the 16-byte
// chunk c of row r sits at slot c ^ (4 (r & 3)). A transposing operand read
// serves 32 lanes per LDS cycle: two 16-lane groups, each reading 4
// consecutive token rows x 32 bytes, 16 channels apart. With this swizzle the
// 16 chunks they touch fall in 16 distinct 16-byte bank groups.
__device__ inline int swz(int r) { return 4 * (r & 3); }

// LDS DMA: lane l's 16 bytes at gptr land at LDS byte address lds_addr + 16 l
// (lds_addr is wave-uniform).
// Issued through asm so the compiler does not wait for it before unrelated LDS
// reads; completion is awaited explicitly with s_waitcnt vmcnt.
__device__ inline void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ inline v4i16 tr16(const char* lds_generic, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)(lds_generic) + off));
}

template <int MODE>
__device__ inline void tile_loop(const uint16_t* srcA, const uint16_t* srcB, int64_t ld,
                                 int64_t width, int64_t I0, int64_t J0, int64_t t_begin,
                                 int64_t t_end, char* lds, f32x16 (&acc)[4][4]) {
  constexpr int NOP = MODE == M_DIAG ? 1 : 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = (w >> 1) * 128;
  const int wn = (w & 1) * 128;
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(lds));

  // ---- per-lane operand read offsets (within one operand stage)
  // lane = 16 g + 4 q + a: reads token row 8(g >> 1) + q (+ 16 ks + 4 h) and
  // channels c + 4a of 16-channel group c = 16 (g & 1) + 32 i + wm
  const int g = lane >> 4, q = (lane >> 2) & 3, a = lane & 3;
  const int rlane = 8 * (g >> 1) + q;
  int offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chA = wm + 32 * i + 16 * (g & 1) + 4 * a;
    const int chB = wn + 32 * i + 16 * (g & 1) + 4 * a;
    // token rows 16 ks + 4 h + rlane all have (row & 3) == q, hence one swizzle
    offA[i] = rlane * ROWB + (((chA >> 3) ^ swz(rlane)) << 4) + ((chA & 7) << 1);
    offB[i] = rlane * ROWB + (((chB >> 3) ^ swz(rlane)) << 4) + ((chB & 7) << 1);
  }

  // fragments of one 16-token k-step: 4 A and 4 B operands (8 bf16 per lane)
  struct Frags {
    bf16x8 a[4], b[4];
  };
  auto read = [&](Frags& f, int slot, int ks) {
    const char* Ab = lds + slot * NOP * STB;
    const char* Bb = MODE == M_DIAG ? Ab : Ab + STB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i16 lo = tr16(Ab, offA[i] + (16 * ks) * ROWB);
      const v4i16 hi = tr16(Ab, offA[i] + (16 * ks + 4) * ROWB);
      f.a[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i16 lo = tr16(Bb, offB[j] + (16 * ks) * ROWB);
      const v4i16 hi = tr16(Bb, offB[j] + (16 * ks + 4) * ROWB);
      f.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // interleave: the next k-step's sixteen LDS reads two per MFMA over the
  // first eight MFMAs, so they have landed before the next group starts
  auto interleave = [&]() {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // ---- DMA addressing: wave w fills rows 8w..8w+7 of each operand stage with
  // 4 instructions of 2 rows; lane l -> row (l >> 5), slot (l & 31) holding
  // global chunk (l & 31) ^ swz(row)
  const int dr = lane >> 5;
  const int dslot = lane & 31;
  const uint16_t* gA[4];
  const uint16_t* gB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * w + 2 * j + dr;
    const int c = dslot ^ swz(r);
    const int64_t chA = min(I0 + 8 * c, width - 8);
    const int64_t chB = min(J0 + 8 * c, width - 8);
    gA[j] = srcA + (t_begin + r) * ld + chA;
    gB[j] = srcB + (t_begin + r) * ld + chB;
  }
  auto issue = [&](int64_t stage, int slot) {
    const int64_t off = stage * KS * ld;
    const uint32_t sb = lds_base + uint32_t(slot * NOP * STB);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(gA[j] + off, sb + uint32_t((8 * w + 2 * j) * ROWB));
    if (MODE != M_DIAG) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(gB[j] + off, sb + STB + uint32_t((8 * w + 2 * j) * ROWB));
    }
  };

  const int64_t n_full = (t_end - t_begin) / KS;
  const int tail = int((t_end - t_begin) - n_full * KS);

  // ---- partial last stage: ordinary loads with zero fill, processed first
  if (tail > 0) {
    const int r = t >> 3;               // token row 0..31
    const int c0 = (t & 7) * 4;         // 4 chunks per thread
    const int64_t tok = t_begin + n_full * KS + r;
    const bool ok = r < tail;
    const int64_t tr_ = ok ? tok : t_begin + n_full * KS;
#pragma unroll
    for (int op = 0; op < NOP; ++op) {
      const uint16_t* src = op == 0 ? srcA : srcB;
      const int64_t c0g = op == 0 ? I0 : J0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + k;
        const int64_t ch = min(c0g + 8 * c, width - 8);
        uint4 v = *reinterpret_cast<const uint4*>(src + tr_ * ld + ch);
        if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(lds + op * STB + r * ROWB + ((c ^ swz(r)) << 4)) = v;
      }
    }
    __syncthreads();
    Frags f0, f1;
    read(f0, 0, 0);
    read(f1, 0, 1);
    mma(f0);
    mma(f1);
    __syncthreads();
  }
  if (n_full == 0) return;

  // ---- full stages through the DMA ring (KS = 2 k-steps per stage, NST
  // slots, stage s in slot s % NST). Iteration s: the MFMAs of k-step 0 run
  // while the k-step 1 operands of stage s are read; stage s+1 is awaited
  // (own DMA: vmcnt; other waves: the barrier, which also retires every read
  // of slot s); stage s+NST is issued into slot s; the MFMAs of k-step 1 run
  // while stage s+1's k-step 0 operands are read. NST - 1 stages stay in
  // flight behind the one being consumed.
  constexpr int PER = 4 * NOP;  // DMA instructions per stage per wave
  auto wait_stages = [&](int64_t k) {  // at most k stages may stay outstanding
    if (k >= 3) wait_vm<3 * PER>();
    else if (k == 2) wait_vm<2 * PER>();
    else if (k == 1) wait_vm<PER>();
    else wait_vm<0>();
  };
  static_assert(NST <= 4, "wait_stages covers at most 3 outstanding stages");
  for (int k = 0; k < NST; ++k)
    if (k < n_full) issue(k, k);
  wait_stages(min<int64_t>(n_full, NST) - 1);
  __syncthreads();
  Frags f0, f1;
  read(f0, 0, 0);
  int slot = 0;
  for (int64_t s = 0; s + 1 < n_full; ++s) {
    const int nslot = slot + 1 == NST ? 0 : slot + 1;
    read(f1, slot, 1);
    mma(f0);
    interleave();
    wait_stages(min<int64_t>(n_full, s + NST) - (s + 2));
    __syncthreads();
    if (s + NST < n_full) issue(s + NST, slot);
    read(f0, nslot, 0);
    mma(f1);
    interleave();
    slot = nslot;
  }
  read(f1, slot, 1);
  mma(f0);
  mma(f1);
}

__global__ __launch_bounds__(256) void cov_bf16_kernel(CovArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const CovItem it = a.items[blockIdx.x];
  if (it.kind < 0) return;
  const int kind = it.kind, I = it.I, J = it.J;
  const uint16_t* srcB = kind == K_HG ? a.G : a.Xq;
  const uint16_t* srcA = kind == K_D ? a.dX : srcB;
  const int64_t width = kind == K_HG ? a.d_out : a.d_in;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = (w >> 1) * 128;
  const int wn = (w & 1) * 128;
  const int lr = lane & 31;
  const int lk = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (it.t0 < it.t1) {
    const int64_t I0 = int64_t(I) * CT, J0 = int64_t(J) * CT;
    if (kind != K_D && I == J)
      tile_loop<M_DIAG>(srcA, srcB, width, width, I0, J0, it.t0, it.t1, lds, acc);
    else
      tile_loop<M_PAIR>(srcA, srcB, width, width, I0, J0, it.t0, it.t1, lds, acc);
  }

  // acc[i][j][r] holds C[I*CT + wm + 32i + 8(r/4) + 4lk + r%4][J*CT + wn + 32j + lr]
  if (it.slot < 0) {
    const int64_t dim = width;
    const int64_t row0 = int64_t(I) * CT + wm;
    const int64_t col0 = int64_t(J) * CT + wn;
    float* C = a.out[kind];
    const float alpha = a.alpha, beta = a.beta;
    const bool mirror = (kind != K_D) && (I != J);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t m = row0 + 32 * i + 8 * q + 4 * lk;  // first of 4 consecutive rows
          const int64_t n = col0 + 32 * j + lr;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][4 * q + e];
          if (n < dim) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (m + e < dim) {
                float o = v[e];
                if (beta != 0.f) o += beta * C[(m + e) * dim + n];
                C[(m + e) * dim + n] = o;
              }
            }
            if (mirror && m + 3 < dim) {  // transposed copy: row n, columns m..m+3
              float4* p = reinterpret_cast<float4*>(C + n * dim + m);
              float4 o = make_float4(v[0], v[1], v[2], v[3]);
              if (beta != 0.f) {
                const float4 old = *p;
                o.x += beta * old.x;
                o.y += beta * old.y;
                o.z += beta * old.z;
                o.w += beta * old.w;
              }
              *p = o;
            }
          }
        }
  } else {
    // partial tile, row-major 256 x 256 in its slot
    float* P = a.pool + it.slot * int64_t(CT * CT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int n = wn + 32 * j + lr;
          P[m * CT + n] = acc[i][j][r];
        }
  }
}

constexpr size_t COV_LDS = size_t(NST) * 2 * STB;  // 128 KB

// dX = bf16_rne(X - Xq), 8 elements per thread (16-byte loads and stores);
// the packed fp32 -> bf16 conversion rounds to nearest even.
__device__ inline uint32_t drift2(uint32_t x, uint32_t q) {
  const f32x2 va = {__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u)};
  const f32x2 vb = {__uint_as_float(q << 16), __uint_as_float(q & 0xFFFF0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(va - vb, bf16x2));
}

__global__ __launch_bounds__(256) void drift_bf16_kernel(const uint4* __restrict__ X,
                                                         const uint4* __restrict__ Xq,
                                                         uint4* __restrict__ dX, int64_t n8) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += int64_t(gridDim.x) * 256) {
    const uint4 x = X[i], q = Xq[i];
    dX[i] = make_uint4(drift2(x.x, q.x), drift2(x.y, q.y), drift2(x.z, q.z), drift2(x.w, q.w));
  }
}

// Sum the pool slots of one tile in slot order, apply alpha/beta, write the
// tile and, for off-diagonal tiles of H_X and H_G, its transpose. One
// workgroup per 64 x 64 sub-block of a 256 x 256 tile; each thread sums four
// float4 of it, with the loads of four slots in flight together (the sum of
// every element still runs over the slots in order: deterministic).
__global__ __launch_bounds__(256) void cov_pool_reduce_kernel(const CovRed* __restrict__ reds,
                                                              const float* __restrict__ pool,
                                                              float* HX, float* D, float* HG,
                                                              int64_t d_in, int64_t d_out,
                                                              float alpha, float beta) {
  __shared__ float tileT[64][65];
  const CovRed rd = reds[blockIdx.x >> 4];
  const int sub = blockIdx.x & 15;
  float* C = rd.kind == K_HX ? HX : rd.kind == K_D ? D : HG;
  const int64_t dim = rd.kind == K_HG ? d_out : d_in;
  const int lr0 = (sub >> 2) * 64, lc0 = (sub & 3) * 64;
  const int t = threadIdx.x;
  const int c4 = 4 * (t & 15);  // column within the sub-block
  const int rq = t >> 4;        // rows rq + 16 h
  const float* base = pool + rd.slot0 * int64_t(CT * CT) + lr0 * CT + lc0 + c4;
  float4 acc[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < rd.count; k0 += 4) {
    float4 v[4][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int h = 0; h < 4; ++h)
        v[kk][h] = k0 + kk < rd.count
                       ? *reinterpret_cast<const float4*>(base + int64_t(k0 + kk) * CT * CT + (rq + 16 * h) * CT)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (k0 + kk >= rd.count) break;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[h].x += v[kk][h].x;
        acc[h].y += v[kk][h].y;
        acc[h].z += v[kk][h].z;
        acc[h].w += v[kk][h].w;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int rr = rq + 16 * h;
    const int64_t r = int64_t(rd.I) * CT + lr0 + rr;
    const float sv[4] = {alpha * acc[h].x, alpha * acc[h].y, alpha * acc[h].z, alpha * acc[h].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = int64_t(rd.J) * CT + lc0 + c4 + e;
      if (r < dim && c < dim) {
        float o = sv[e];
        if (beta != 0.f) o += beta * C[r * dim + c];
        C[r * dim + c] = o;
      }
      tileT[rr][c4 + e] = sv[e];
    }
  }
  if (rd.kind == K_D || rd.I == rd.J) return;
  __syncthreads();
  // transpose: element (J*CT + lc0 + rr, I*CT + lr0 + tx) = tile[tx][rr]
  const int tx = t & 63;
  const int ty = t >> 6;  // 0..3
  const int64_t c2 = int64_t(rd.I) * CT + lr0 + tx;
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t r2 = int64_t(rd.J) * CT + lc0 + rr;
    if (r2 < dim && c2 < dim) {
      float o = tileT[tx][rr];
      if (beta != 0.f) o += beta * C[r2 * dim + c2];
      C[r2 * dim + c2] = o;
    }
  }
}

// fp32 drift: dX = X - Xq
__global__ void drift_f32_kernel(const float* __restrict__ X, const float* __restrict__ Xq,
                                 float* __restrict__ dX, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dX[i] = X[i] - Xq[i];
}

// ------------------------------------------------------------ schedule

constexpr int XCDS = 8;       // workgroup b runs on XCD b % 8
constexpr int XCD_CUS = 32;   // CUs per XCD: one round of items per XCD
constexpr int GROUP = 32;     // tiles per group (one round on one XCD)
constexpr int64_t MIN_PIECE = 4 * KS;  // shortest token piece of the last round

struct Tile {
  int kind, I, J;
};

// Tiles in bands of 8 tile rows; inside a band column by column, so 32
// consecutive tiles form an 8 x 4 block (lower: clipped at the diagonal).
void band_order(std::vector<Tile>& out, int kind, int nt, bool lower) {
  for (int u0 = 0; u0 < nt; u0 += 8) {
    const int u1 = std::min(u0 + 8, nt);
    const int jn = lower ? u1 : nt;
    for (int J = 0; J < jn; ++J)
      for (int I = lower ? std::max(u0, J) : u0; I < u1; ++I) out.push_back({kind, I, J});
  }
}

struct CovSchedule {
  std::vector<CovItem> items;  // by blockIdx
  std::vector<CovRed> reds;    // tiles with partials
  int64_t slots = 0;
};

int choose_split(int64_t tiles) {
  // One token range per tile when the tiles fill at least one round of the
  // chip (the last round is balanced by pieces); smaller problems split the
  // tokens for at least ~4 items per CU, at most 8 ways.
  if (tiles >= XCDS * XCD_CUS) return 1;
  int s = 1;
  while (s < 8 && tiles * s < 1024) s *= 2;
  return s;
}

CovSchedule build_schedule(int64_t n_tok, int64_t d_in, int64_t d_out, bool hx, bool d, bool hg) {
  std::vector<Tile> tiles;
  const int ti = int(cdiv(d_in, CT)), to = int(cdiv(d_out, CT));
  if (hx) band_order(tiles, K_HX, ti, true);
  if (d) band_order(tiles, K_D, ti, false);
  if (hg) band_order(tiles, K_HG, to, true);
  CovSchedule S;
  const int64_t T = int64_t(tiles.size());
  if (T == 0) return S;
  int ns = choose_split(T);
  while (ns > 1 && cdiv(n_tok, ns) < KS) ns /= 2;
  const int64_t chunk = cdiv(cdiv(n_tok, ns), KS) * KS;
  auto range = [&](int s, int64_t& t0, int64_t& t1) {
    t0 = std::min<int64_t>(n_tok, s * chunk);
    t1 = std::min<int64_t>(n_tok, t0 + chunk);
  };
  const int64_t G = cdiv(T, GROUP);
  const int64_t Q = G * ns;          // group-splits
  const int64_t R = Q / XCDS;        // full rounds
  struct Raw {
    int tile;
    int64_t t0, t1;
  };
  std::vector<Raw> raw;  // by blockIdx, tile -1 = idle
  raw.assign(size_t(R * XCDS * XCD_CUS), Raw{-1, 0, 0});
  for (int64_t j = 0; j < R * XCDS; ++j) {
    const int64_t g = j / ns;
    const int s = int(j % ns);
    const int64_t x = j % XCDS, round = j / XCDS;
    for (int k = 0; k < GROUP; ++k) {
      const int64_t tile = g * GROUP + k;
      if (tile >= T) continue;
      Raw r{int(tile), 0, 0};
      range(s, r.t0, r.t1);
      raw[size_t(XCDS * (round * XCD_CUS + k) + x)] = r;
    }
  }
  // last partial round: cut the remaining items into pieces over every CU
  std::vector<Raw> left;
  for (int64_t j = R * XCDS; j < Q; ++j) {
    const int64_t g = j / ns;
    const int s = int(j % ns);
    for (int k = 0; k < GROUP; ++k) {
      const int64_t tile = g * GROUP + k;
      if (tile >= T) continue;
      Raw r{int(tile), 0, 0};
      range(s, r.t0, r.t1);
      left.push_back(r);
    }
  }
  if (!left.empty()) {
    const int64_t L = int64_t(left.size());
    const int64_t len = left[0].t1 - left[0].t0;
    int64_t f = std::max<int64_t>(1, (XCDS * XCD_CUS) / L);
    f = std::max<int64_t>(1, std::min<int64_t>(f, len / MIN_PIECE));
    const int64_t plen = cdiv(cdiv(len, f), KS) * KS;
    std::vector<Raw> pieces;
    for (const Raw& r : left)
      for (int64_t p = 0; p < f; ++p) {
        const int64_t t0 = std::min(r.t1, r.t0 + p * plen);
        const int64_t t1 = std::min(r.t1, t0 + plen);
        if (t0 < t1 || p == 0) pieces.push_back(Raw{r.tile, t0, t1});
      }
    // piece q -> XCD q % 8, in order within each XCD
    const int64_t base = int64_t(raw.size());
    const int64_t nrow = cdiv(int64_t(pieces.size()), XCDS);
    raw.resize(size_t(base + nrow * XCDS), Raw{-1, 0, 0});
    for (int64_t q = 0; q < int64_t(pieces.size()); ++q) raw[size_t(base + q)] = pieces[size_t(q)];
  }
  // items per tile: direct if one item covers all tokens, else pool slots
  std::vector<std::vector<int64_t>> per_tile(static_cast<size_t>(T));
  for (int64_t b = 0; b < int64_t(raw.size()); ++b)
    if (raw[size_t(b)].tile >= 0) per_tile[size_t(raw[size_t(b)].tile)].push_back(b);
  S.items.assign(raw.size(), CovItem{-1, 0, 0, -1, 0, 0});
  for (int64_t tix = 0; tix < T; ++tix) {
    const Tile& tl = tiles[size_t(tix)];
    const auto& bs = per_tile[size_t(tix)];
    const bool direct = bs.size() == 1 && raw[size_t(bs[0])].t0 == 0 && raw[size_t(bs[0])].t1 == n_tok;
    if (!direct) S.reds.push_back(CovRed{tl.kind, tl.I, tl.J, int32_t(bs.size()), S.slots});
    for (int64_t b : bs) {
      const Raw& r = raw[size_t(b)];
      S.items[size_t(b)] = CovItem{tl.kind, tl.I, tl.J, direct ? -1 : int32_t(S.slots++), r.t0, r.t1};
    }
  }
  return S;
}

// The schedule depends only on the shapes and on which outputs are asked for.
// Building it takes a few hundred microseconds of host time (as long as the
// kernels of a small token chunk), so the last one built is kept per thread.
const CovSchedule& schedule_for(int64_t n_tok, int64_t d_in, int64_t d_out, bool hx, bool d,
                                bool hg) {
  struct Cache {
    bool valid = false;
    int64_t n_tok = 0, d_in = 0, d_out = 0;
    bool hx = false, d = false, hg = false;
    CovSchedule S;
  };
  thread_local Cache c;
  if (!c.valid || c.n_tok != n_tok || c.d_in != d_in || c.d_out != d_out || c.hx != hx ||
      c.d != d || c.hg != hg) {
    c.valid = false;
    c.S = build_schedule(n_tok, d_in, d_out, hx, d, hg);
    c.n_tok = n_tok;
    c.d_in = d_in;
    c.d_out = d_out;
    c.hx = hx;
    c.d = d;
    c.hg = hg;
    c.valid = true;
  }
  return c.S;
}

size_t sched_bytes(const CovSchedule& S) {
  Arena ar{nullptr, 0, 0};
  ar.take<CovItem>(S.items.size());
  ar.take<CovRed>(S.reds.size());
  ar.take<float>(size_t(S.slots) * CT * CT);
  return ar.used;
}

}  // namespace

size_t cov_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out, kq_dtype dt, bool hx, bool d,
                    bool hg) {
  Arena ar{nullptr, 0, 0};
  if (dt == KQ_F32) {
    if (d) ar.take<float>(size_t(n_tok) * d_in);
    return ar.used;
  }
  if (d) ar.take<uint16_t>(size_t(n_tok) * d_in);  // bf16 drift
  return ar.used + 256 + sched_bytes(schedule_for(n_tok, d_in, d_out, hx, d, hg));
}

kq_status cov_run(const void* X, const void* Xq, const void* G, kq_dtype dt, int64_t n_tok,
                  int64_t d_in, int64_t d_out, float alpha, float beta, float* HX, float* D,
                  float* HG, Arena& ws, hipStream_t s) {
  if (dt == KQ_F32) {
    const float* x = static_cast<const float*>(X);
    const float* xq = static_cast<const float*>(Xq);
    const float* g = static_cast<const float*>(G);
    KQ_TRY(mark_kernel(KQ_OP_ACCUMULATE_COV, 0, s));
    if (HX) {
      GemmArgs a = gemm_args(xq, d_in, xq, d_in, HX, d_in, d_in, d_in, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    if (D) {
      float* dx = ws.take<float>(size_t(n_tok) * d_in);
      if (!dx) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
      const int64_t n = n_tok * d_in;
      drift_f32_kernel<<<unsigned(std::min<int64_t>(cdiv(n, 256), 8192)), 256, 0, s>>>(x, xq, dx, n);
      KQ_HIP(hipGetLastError());
      GemmArgs a = gemm_args(dx, d_in, xq, d_in, D, d_in, d_in, d_in, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    if (HG) {
      GemmArgs a = gemm_args(g, d_out, g, d_out, HG, d_out, d_out, d_out, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    return mark_kernel(KQ_OP_ACCUMULATE_COV, 1, s);
  }

  const CovSchedule& S = schedule_for(n_tok, d_in, d_out, HX != nullptr, D != nullptr, HG != nullptr);
  if (S.items.empty()) return KQ_OK;
  CovArgs a{};
  a.Xq = static_cast<const uint16_t*>(Xq);
  uint16_t* dx = nullptr;
  if (D) {
    dx = ws.take<uint16_t>(size_t(n_tok) * d_in);
    if (!dx) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
  }
  CovItem* items = ws.take<CovItem>(S.items.size());
  CovRed* reds = ws.take<CovRed>(S.reds.size());
  float* pool = ws.take<float>(size_t(S.slots) * CT * CT);
  if (!items || (!S.reds.empty() && !reds) || (S.slots && !pool))
    return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
  // the schedule goes up first: a copy from pageable memory can hold the
  // host until the stream reaches it, and ahead of the drift pass that wait
  // does not leave the kernels behind it unlaunched
  KQ_HIP(hipMemcpyAsync(items, S.items.data(), S.items.size() * sizeof(CovItem),
                        hipMemcpyHostToDevice, s));
  if (!S.reds.empty())
    KQ_HIP(hipMemcpyAsync(reds, S.reds.data(), S.reds.size() * sizeof(CovRed),
                          hipMemcpyHostToDevice, s));
  if (D) {
    const int64_t n8 = n_tok * d_in / 8;
    drift_bf16_kernel<<<unsigned(std::min<int64_t>(cdiv(n8, 256), 16384)), 256, 0, s>>>(
        static_cast<const uint4*>(X), static_cast<const uint4*>(Xq), reinterpret_cast<uint4*>(dx), n8);
    KQ_HIP(hipGetLastError());
    a.dX = dx;
  }
  a.G = static_cast<const uint16_t*>(G);
  a.d_in = d_in;
  a.d_out = d_out;
  a.alpha = alpha;
  a.beta = beta;
  a.out[0] = HX;
  a.out[1] = D;
  a.out[2] = HG;
  a.items = items;
  a.pool = pool;
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(cov_bf16_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(COV_LDS)));
  KQ_TRY(mark_kernel(KQ_OP_ACCUMULATE_COV, 0, s));
  cov_bf16_kernel<<<unsigned(S.items.size()), 256, COV_LDS, s>>>(a);
  KQ_HIP(hipGetLastError());
  KQ_TRY(mark_kernel(KQ_OP_ACCUMULATE_COV, 1, s));
  if (!S.reds.empty()) {
    cov_pool_reduce_kernel<<<unsigned(S.reds.size() * 16), 256, 0, s>>>(reds, pool, HX, D, HG, d_in,
                                                                     d_out, alpha, beta);
    KQ_HIP(hipGetLastError());
  }
  return KQ_OK;
}

}  // namespace kq
