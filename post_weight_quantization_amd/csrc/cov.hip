// Stage 1: covariances H_X = Xq^T Xq, D = dX^T Xq, H_G = G^T G (scaled by alpha).
//
// KronQ summary (hyper.ai), Method: the Fisher of a linear layer factors under
// K-FAC as H ~ H_X (x) H_G with H_X = E[x x^T] and H_G = E[g g^T]; the GPTAQ
// objective adds the drift term dX X^T. With token-major inputs (one token
// per row), each output is a "TN" product C[i][j] = sum_t A[t][i] B[t][j].
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * one launch covers every output tile of all three matrices (H_X and H_G
//     lower-triangle tiles only, D full), times `nsplit` token splits;
//     blockIdx % nsplit selects the split so that, with nsplit | 8, all
//     workgroups on one XCD stream the same token range through its L2;
//   * workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 MFMA blocks,
//     256 accumulator registers per lane), 64 tokens per LDS stage, two
//     stages of LDS (128 KB) with the next stage's global loads in flight
//     while the current one feeds the MFMAs;
//   * each thread loads 8 tokens x 8 channels (16 bytes per token row, 32
//     threads cover a 512-byte row segment) and transposes them in registers
//     with v_perm so LDS holds [channel][token]; an MFMA operand (8
//     consecutive tokens of one channel) is then one 16-byte LDS read. The
//     16-byte chunks of each channel row are XOR-swizzled so the transposed
//     stores and the operand reads are both bank-conflict free;
//   * for D the A operand is formed on the fly: dX = bf16_rne(X - Xq), the
//     rounding done by the packed fp32->bf16 conversion (nearest even);
//   * with nsplit == 1 the epilogue applies alpha/beta and mirrors the lower
//     tiles of H_X and H_G into the upper triangle; otherwise partial sums go
//     to scratch and a reduction kernel does the same.
// fp32 path (small workloads): the generic fp32 MFMA GEMM with transposed A.
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

struct CovArgs {
  const uint16_t* Xq;
  const uint16_t* dX;  // bf16 drift, token-major (written by the drift pre-pass)
  const uint16_t* G;
  int64_t n_tok, d_in, d_out;
  float alpha, beta;
  float* out[3];       // final outputs (direct mode)
  float* part;         // partial sums (split mode): [split][HX | D | HG]
  int64_t part_stride; // floats per split
  int64_t part_off[3]; // offset of each matrix inside one split
  int nt_in, nt_out;   // tiles per dimension
  int tasks[3];        // tiles per matrix (0 when skipped)
  int nsplit;
  int64_t tok_chunk;   // tokens per split (multiple of KS)
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ inline void tri_decode(int t, int& I, int& J) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

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
  // interleave: one MFMA, one LDS read, sixteen times
  auto interleave = [&]() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
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

  // ---- full stages through the DMA ring (KS = 2 k-steps per stage).
  // Stage s: MFMAs of k-step 0 run while k-step 1 operands are read; then the
  // data of stage s+1 is awaited (own DMA: vmcnt; other waves: barrier), the
  // DMA of stage s+3 is issued into the slot stage s-1 used, and the MFMAs of
  // k-step 1 run while stage s+1's k-step 0 operands are read.
  constexpr int PER = 4 * NOP;  // DMA instructions per stage per wave
  for (int k = 0; k < NST - 1; ++k)
    if (k < n_full) issue(k, k);
  if (n_full >= 3) wait_vm<2 * PER>();
  else if (n_full == 2) wait_vm<PER>();
  else wait_vm<0>();
  __syncthreads();
  Frags f0, f1;
  read(f0, 0, 0);
  for (int64_t s = 0; s + 1 < n_full; ++s) {
    read(f1, int(s % NST), 1);
    mma(f0);
    interleave();
    if (s + 2 < n_full) wait_vm<PER>();
    else wait_vm<0>();
    __syncthreads();
    if (s + 3 < n_full) issue(s + 3, int((s + 3) % NST));
    read(f0, int((s + 1) % NST), 0);
    mma(f1);
    interleave();
  }
  read(f1, int((n_full - 1) % NST), 1);
  mma(f0);
  mma(f1);
}

__global__ __launch_bounds__(256) void cov_bf16_kernel(CovArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int b = blockIdx.x;
  const int split = b % a.nsplit;
  int tile = b / a.nsplit;
  int kind, I, J;
  if (tile < a.tasks[0]) {
    kind = K_HX;
    tri_decode(tile, I, J);
  } else if ((tile -= a.tasks[0]) < a.tasks[1]) {
    kind = K_D;
    I = tile / a.nt_in;
    J = tile % a.nt_in;
  } else {
    tile -= a.tasks[1];
    kind = K_HG;
    tri_decode(tile, I, J);
  }
  const uint16_t* srcB = kind == K_HG ? a.G : a.Xq;
  const uint16_t* srcA = kind == K_D ? a.dX : srcB;
  const int64_t width = kind == K_HG ? a.d_out : a.d_in;

  const int64_t t_begin = int64_t(split) * a.tok_chunk;
  const int64_t t_end = min(a.n_tok, t_begin + a.tok_chunk);

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

  if (t_begin < t_end) {
    const int64_t I0 = int64_t(I) * CT, J0 = int64_t(J) * CT;
    if (kind != K_D && I == J)
      tile_loop<M_DIAG>(srcA, srcB, width, width, I0, J0, t_begin, t_end, lds, acc);
    else
      tile_loop<M_PAIR>(srcA, srcB, width, width, I0, J0, t_begin, t_end, lds, acc);
  }

  // acc[i][j][r] holds C[I*CT + wm + 32i + 8(r/4) + 4lk + r%4][J*CT + wn + 32j + lr]
  const int64_t dim = width;
  const int64_t row0 = int64_t(I) * CT + wm;
  const int64_t col0 = int64_t(J) * CT + wn;
  if (a.nsplit == 1) {
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
    float* P = a.part + split * a.part_stride + a.part_off[kind];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = row0 + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t n = col0 + 32 * j + lr;
          if (m < dim && n < dim) P[m * dim + n] = acc[i][j][r];
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

// Sum the split partials of one matrix, apply alpha/beta, mirror lower tiles
// of symmetric outputs. 64 x 64 tiles; for symmetric matrices only lower
// tiles are scheduled and each writes both (I, J) and (J, I).
__global__ __launch_bounds__(256) void cov_reduce_kernel(const float* __restrict__ part,
                                                         int64_t part_stride, int nsplit,
                                                         float* C, int64_t dim, float alpha,
                                                         float beta, int sym, int ntile) {
  __shared__ float tileT[64][65];
  int I, J;
  if (sym) {
    tri_decode(blockIdx.x, I, J);
  } else {
    I = blockIdx.x / ntile;
    J = blockIdx.x % ntile;
  }
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;  // 0..3
  const int64_t c = int64_t(J) * 64 + tx;
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t r = int64_t(I) * 64 + rr;
    float s = 0.f;
    if (r < dim && c < dim) {
      for (int k = 0; k < nsplit; ++k) s += part[k * part_stride + r * dim + c];
      float o = alpha * s;
      if (beta != 0.f) o += beta * C[r * dim + c];
      C[r * dim + c] = o;
      s = alpha * s;
    }
    tileT[rr][tx] = s;
  }
  if (!sym || I == J) return;
  __syncthreads();
  // write the transpose: element (J*64 + rr, I*64 + tx) = tile[tx][rr]
  const int64_t c2 = int64_t(I) * 64 + tx;
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t r2 = int64_t(J) * 64 + rr;
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

int choose_split(int tiles) {
  // Aim for >= ~4 workgroups per CU (256 CUs); splits stay a divisor of the 8 XCDs.
  int s = 1;
  while (s < 8 && tiles * s < 1024) s *= 2;
  return s;
}

int cov_tiles(int64_t d_in, int64_t d_out, bool hx, bool d, bool hg) {
  const int64_t ti = cdiv(d_in, CT), to = cdiv(d_out, CT);
  int64_t n = 0;
  if (hx) n += ti * (ti + 1) / 2;
  if (d) n += ti * ti;
  if (hg) n += to * (to + 1) / 2;
  return int(n);
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
  const int tiles = cov_tiles(d_in, d_out, hx, d, hg);
  const int ns = choose_split(tiles);
  if (ns > 1) {
    const size_t per = (hx ? d_in * d_in : 0) + (d ? d_in * d_in : 0) + (hg ? d_out * d_out : 0);
    ar.take<float>(per * ns);
  }
  return ar.used;
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

  CovArgs a{};
  a.Xq = static_cast<const uint16_t*>(Xq);
  if (D) {
    uint16_t* dx = ws.take<uint16_t>(size_t(n_tok) * d_in);
    if (!dx) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
    const int64_t n8 = n_tok * d_in / 8;
    drift_bf16_kernel<<<unsigned(std::min<int64_t>(cdiv(n8, 256), 16384)), 256, 0, s>>>(
        static_cast<const uint4*>(X), static_cast<const uint4*>(Xq), reinterpret_cast<uint4*>(dx), n8);
    KQ_HIP(hipGetLastError());
    a.dX = dx;
  }
  a.G = static_cast<const uint16_t*>(G);
  a.n_tok = n_tok;
  a.d_in = d_in;
  a.d_out = d_out;
  a.alpha = alpha;
  a.beta = beta;
  a.out[0] = HX;
  a.out[1] = D;
  a.out[2] = HG;
  a.nt_in = int(cdiv(d_in, CT));
  a.nt_out = int(cdiv(d_out, CT));
  a.tasks[0] = HX ? a.nt_in * (a.nt_in + 1) / 2 : 0;
  a.tasks[1] = D ? a.nt_in * a.nt_in : 0;
  a.tasks[2] = HG ? a.nt_out * (a.nt_out + 1) / 2 : 0;
  const int tiles = a.tasks[0] + a.tasks[1] + a.tasks[2];
  if (tiles == 0) return KQ_OK;
  int ns = choose_split(tiles);
  // each split needs at least one stage of tokens
  while (ns > 1 && cdiv(n_tok, ns) < KS) ns /= 2;
  a.nsplit = ns;
  a.tok_chunk = cdiv(cdiv(n_tok, ns), KS) * KS;
  if (ns > 1) {
    int64_t off = 0;
    a.part_off[0] = off;
    if (HX) off += d_in * d_in;
    a.part_off[1] = off;
    if (D) off += d_in * d_in;
    a.part_off[2] = off;
    if (HG) off += d_out * d_out;
    a.part_stride = off;
    a.part = ws.take<float>(size_t(off) * ns);
    if (!a.part) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
  }
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(cov_bf16_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(COV_LDS)));
  KQ_TRY(mark_kernel(KQ_OP_ACCUMULATE_COV, 0, s));
  cov_bf16_kernel<<<unsigned(tiles * ns), 256, COV_LDS, s>>>(a);
  KQ_HIP(hipGetLastError());
  KQ_TRY(mark_kernel(KQ_OP_ACCUMULATE_COV, 1, s));
  if (ns > 1) {
    float* outs[3] = {HX, D, HG};
    const int64_t dims[3] = {d_in, d_in, d_out};
    for (int k = 0; k < 3; ++k) {
      if (!outs[k]) continue;
      const int nt = int(cdiv(dims[k], 64));
      const int sym = k != 1;
      const int blocks = sym ? nt * (nt + 1) / 2 : nt * nt;
      cov_reduce_kernel<<<unsigned(blocks), 256, 0, s>>>(a.part + a.part_off[k], a.part_stride, ns,
                                                         outs[k], dims[k], alpha, beta, sym, nt);
      KQ_HIP(hipGetLastError());
    }
  }
  return KQ_OK;
}

}  // namespace kq
