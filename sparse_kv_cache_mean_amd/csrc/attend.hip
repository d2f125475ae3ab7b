// attend.hip - sparse GQA decode attention over recalled blocks
// (kvoff_sparse_decode).
//
// The pages describe the attention only as SoloHead-aligned sparse attention
// over the paged KV pool ("PulseInfer Guide", aiFetchly, architecture
// figure, section "PulseInfer Architectural Foundations").  What is computed:
//   o[h] = sum_t softmax_t(scale * <q[h], K[t][g]>) V[t][g],  g = floor(h/G),
// over the valid tokens t of the selected blocks of the request (headwise:
// of the blocks KV head g selected), fp32 accumulation, fp32 output.
//
// Design (split-K flash decoding, one workgroup per (request, KV head,
// split), 4 waves, each wave an independent online-softmax worker over
// `bpw` consecutive selected blocks):
//   K tile  lane (quad, col) loads 16 contiguous bytes of token row
//        t*16 + col at dims m*32 + quad*8 (m = 0..3), so four lanes cover 64
//        contiguous bytes of a row.
//   QK on the matrix cores (MFMA=true): v_mfma_f32_16x16x32_{bf16,f16} with
//        A = that 16-token x 32-dim tile and B = the G query heads of the
//        group (columns >= G repeat the last head; their logits are never
//        stored).  Lane (quad, col) gets the logits of
//        tokens quad*4..quad*4+3 for head col; the running max / sum per head
//        is reduced across the four quads with lane shuffles.
//   QK on the vector ALUs (MFMA=false, G <= 8): v_dot2 over the same tile
//        against the lane's 32 query dims of every head, summed across the
//        four quads; every lane then holds all G heads' logits of its two
//        tokens and the per-head max / sum are reduced across the 16 columns.
//   softmax  log2 domain.
//   PV, G <= 4 (or 16-token blocks): fp32 VALU.  Probabilities go to LDS;
//        lane (token group quad, dim group col) loads 16 bytes of V rows
//        t = quad + 4k and accumulates o[h][8 dims] for all G heads.
//   PV, G >= 8 with MFMA QK and 32-token blocks: on the matrix cores.  The
//        K rows of the QK tiles are loaded in an order that leaves quad q
//        with the logits of the consecutive tokens 8q .. 8q+7, so each lane
//        already holds its row of the A operand P (heads x 32 tokens), split
//        into hi and lo halves of the storage type (fp16: scaled by 2^15).
//        V goes through LDS (rows padded to 132 elements, so the column
//        reads of the four quads fall in different banks) and each lane
//        gathers its B operand column V[8q .. 8q+7][dim]; one MFMA pair per
//        16-dim chunk accumulates o[head][dim] with no cross-quad sum.  At
//        G = 4 the two forms measure the same, and the VALU one stays.
// The four waves merge in LDS; one partial (m, l, o[128]) per (head, split)
// goes to the workspace and combine_kernel merges the splits in fixed split
// order, so results are deterministic.  (Merging in the last-arriving
// workgroup instead needs a device-scope release per workgroup, which on this
// part writes back the L2 that the recall just filled; measured 8x slower.)
#include <cstdlib>
#include <mutex>
#include <vector>

#include "kvoff_internal.h"

// Split partials of kvoff_sparse_decode_noalloc: a file-scope device array
// instead of a caller workspace, one copy per GPU for the life of the
// process.  Host code never uses the name itself (on the host it is only a
// stand-in): its device address comes from hipGetSymbolAddress, once per
// device (kvoff::attend_scratch_address).
static __device__ __align__(256) unsigned char scratch[KVOFF_NOALLOC_SCRATCH_BYTES];

namespace kvoff {

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_dev;  // device address of `scratch`, per device
}  // namespace

int attend_scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0) return fail(KVOFF_EINVAL, "device %d", device);
  if ((int)g_scratch_dev.size() <= device) g_scratch_dev.resize((size_t)device + 1, nullptr);
  if (!g_scratch_dev[device]) {
    int cur = -1;
    KVOFF_HIP(hipGetDevice(&cur));
    if (cur != device) return fail(KVOFF_ESTATE, "device %d is not current (%d is)", device, cur);
    void* p = nullptr;
    KVOFF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(KVOFF_EHIP, "no device address for the attention scratch");
    g_scratch_dev[device] = p;
  }
  *out = g_scratch_dev[device];
  return KVOFF_OK;
}

namespace {

constexpr int ATT_WAVES = 4;
constexpr int MAXB = 8;  // most blocks per wave
constexpr int PART = 2 + kHeadDim;  // m, l, o[128]


typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

struct AttendArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const uint16_t* q;
  const uint8_t* pool;
  const int32_t* table;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  float* part;
  int64_t slice_bytes;
  int64_t n_slices;  // slices the pool holds (n_slots * Hkv); entries at or past it are skipped
  int32_t k_stride, S, bpw, Hq, Hkv, hw;
  float scale_log2;
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack8(uint4 w, float f[8]) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (BF16) {
      f[2 * e] = __uint_as_float(x[e] << 16);
      f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
    } else {
      f[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[e] & 0xffffu));
      f[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[e] >> 16));
    }
  }
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// sum over lanes (a, b, 2 packed values each) of a * b, accumulated into c
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
  }
}

template <int W>  // max / sum over the W lanes of an aligned group (W <= 16)
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <int W>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// G >= 8 with both contractions on the matrix cores fits 3 waves per SIMD
// when asked (G = 8: 160 VGPRs, no spills; left to itself the compiler takes
// more registers and 2 waves).  G = 4 with 32-token blocks fits 4 waves
// unasked (120 + 8 accumulation registers).
template <int G, int BS, bool BF16, bool MFMA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MFMA && BS == 32 && G >= 8 ? 3 : 1)))
void attend_kernel(AttendArgs a) {
  static_assert(MFMA || G <= 8, "the VALU QK keeps every head's query slice in registers");
  static_assert(G <= 16, "one MFMA tile holds the group's heads");
  constexpr int D = kHeadDim;
  constexpr int TILES = BS / 16;
  constexpr int GV = MFMA ? 1 : G;  // heads whose query slice a lane holds (VALU)
  // P V on the matrix cores too (32-token blocks, G >= 8): P (heads x
  // tokens) from registers as the A operand, V (tokens x dims) through LDS as
  // B.  Measured at the Llama-3-8B layer's 128 MiB: G = 16 68.9 -> 30.8 us,
  // G = 8 32.1 -> 28.4 us.  At G = 4 the two forms run within noise of each
  // other (both at 4 waves per SIMD, the MFMA one when asked for it), so G = 4
  // and below keep the simpler VALU P V.
  constexpr bool PVM = MFMA && BS == 32 && G >= 8;
  constexpr int VS = 132;  // LDS row stride of the V tile (elements): column reads hit 4 bank groups
  __shared__ float p_s[ATT_WAVES][PVM ? 1 : BS][G];
  __shared__ float alpha_s[ATT_WAVES][PVM ? 16 : G];
  __shared__ float wm[ATT_WAVES][G], wl[ATT_WAVES][G];
  // the waves' o partials for the final merge; with P V on the matrix cores
  // each wave's share lives in its own V tile (8,448 bytes, at most 8,192
  // needed), which that wave no longer reads once its block loop is done
  __shared__ float wo_s[ATT_WAVES][PVM ? 1 : G][D];
  __shared__ __align__(16) uint16_t v_s[ATT_WAVES][PVM ? BS * VS : 1];
  static_assert(!PVM || G * D * sizeof(float) <= BS * VS * sizeof(uint16_t), "o partials fit the V tile");
  auto wo = [&](int w) -> float* {
    if constexpr (PVM) return reinterpret_cast<float*>(&v_s[w][0]);
    else return &wo_s[w][0][0];
  };

  // grid (split, KV head, request): no index waits for a kernel argument
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform over the wave; saying so puts the wave's block
  // ids, table entries and record addresses in scalar registers (G = 4 with
  // 32-token blocks then fits 128 registers: 4 waves per SIMD, not 3)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = lane >> 4, col = lane & 15;

  // Prologue: two memory round trips before the K/V loads go out.
  //  1. The kernel arguments, all behind one wait (the empty asm statements
  //     are points of use; without them the compiler reads each argument
  //     where it is first needed and waits for each in turn).
  //  2. One vector load in which each lane fetches one of: the wave's block
  //     ids (lanes 0-7) and table entries (8-15), the selection count (16)
  //     and the request's token count (17+).  The indices are clamped inside
  //     the row, since the count is not known yet.  The value stays in its
  //     register, and each block's id and entry are read from it with a
  //     scalar lane select.  (Left to itself the compiler loads these with
  //     scalar loads behind the split test below, one wait each.)
  // The query fragments load after the split test, beside the K/V loads:
  // a split with nothing to do then reads nothing more (the variable-recall
  // layer has thousands of them).  Measured at the Llama-3-8B layer from
  // clean HBM: 0.9-1.2 us less than the chain of dependent loads.
  const int id = a.batch.id[r];
  asm volatile("" ::"s"(a.hw), "s"(a.Hkv), "s"(a.Hq), "s"(a.k_stride), "s"(a.bpw), "s"(a.sel_idx),
               "s"(a.table), "s"(a.sel_cnt), "s"(a.reqs), "s"(a.q), "s"(id));
  const int64_t row = a.hw ? ((int64_t)r * a.Hkv + g) * a.k_stride : (int64_t)r * a.k_stride;
  const int i0 = (s * ATT_WAVES + wave) * a.bpw;
  int sel_n, n_tokens, mv;
  {
    // addresses fixed before the choice, so that it is a per-lane select
    // and not branches
    const int32_t* p_sel = a.sel_idx + row;
    const int32_t* p_tab = a.table + row;
    const int32_t* p_cnt = a.sel_cnt + r;
    const int32_t* p_tok = &a.reqs[id].n_tokens;
    asm volatile("" ::"s"(p_sel), "s"(p_tab), "s"(p_cnt), "s"(p_tok));
    const int i = min(i0 + (lane & (MAXB - 1)), a.k_stride - 1);
    const int32_t* src = lane < MAXB       ? p_sel + i
                         : lane < 2 * MAXB  ? p_tab + i
                         : lane == 2 * MAXB ? p_cnt
                                            : p_tok;
    mv = *src;
    sel_n = __builtin_amdgcn_readlane(mv, 2 * MAXB);
    n_tokens = __builtin_amdgcn_readlane(mv, 2 * MAXB + 1);
  }
  const int cnt = min(sel_n, a.k_stride);
  // a split past the request's selection has nothing to do: it writes no
  // partial, and the combine reads only the splits that hold blocks
  if (s * ATT_WAVES * a.bpw >= cnt) return;  // uniform over the workgroup
  const int i1 = min(i0 + a.bpw, cnt);

  // MFMA: B fragments, query head g*G + col, dims m*32 + quad*8 .. +7.
  // VALU: the same dims of every head of the group.
  uint4 qf[4];
  uint4 qv[GV][4];
  if constexpr (MFMA) {
    // columns col >= G repeat head G-1: MFMA output columns are independent
    // and those columns' logits are never stored, so they need no zeroing
    const uint16_t* qh = a.q + ((int64_t)r * a.Hq + (int64_t)g * G + min(col, G - 1)) * D;
#pragma unroll
    for (int m = 0; m < 4; ++m) qf[m] = *reinterpret_cast<const uint4*>(qh + m * 32 + quad * 8);
  } else {
#pragma unroll
    for (int h = 0; h < GV; ++h) {
      const uint16_t* qh = a.q + ((int64_t)r * a.Hq + (int64_t)g * G + h) * D;
#pragma unroll
      for (int m = 0; m < 4; ++m) qv[h][m] = *reinterpret_cast<const uint4*>(qh + m * 32 + quad * 8);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // MFMA: head col's running max (log2) and sum
  float mh[GV], lh[GV];                  // VALU: every head's
#pragma unroll
  for (int h = 0; h < GV; ++h) {
    mh[h] = -INFINITY;
    lh[h] = 0.f;
  }
  float o[PVM ? 1 : G][8];  // VALU P V: heads x the lane's 8 dims
#pragma unroll
  for (int h = 0; h < (PVM ? 1 : G); ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  // MFMA P V: per 16-dim chunk c, heads quad*4 + i at dim c*16 + col
  f32x4_t oc[PVM ? 8 : 1];
#pragma unroll
  for (int c = 0; c < (PVM ? 8 : 1); ++c) oc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K tile as MFMA A operands / VALU dot operands, V rows for the PV product
  auto load_tiles = [&](const uint16_t* Kp, uint4 (&kf)[TILES][4], uint4 (&vf)[BS / 4]) {
    const uint16_t* Vp = Kp + BS * D;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      // with P V on MFMA, row col of tile t is token 8*(col/4) + 4t + col%4,
      // so that quad q's logits cover the consecutive tokens 8q .. 8q+7
      const int krow = PVM ? 8 * (col >> 2) + 4 * t + (col & 3) : t * 16 + col;
#pragma unroll
      for (int m = 0; m < 4; ++m) kf[t][m] = load16(Kp + krow * D + m * 32 + quad * 8);
    }
#pragma unroll
    for (int k = 0; k < BS / 4; ++k) vf[k] = load16(Vp + (quad + 4 * k) * D + col * 8);
  };
  // one block: logits, online softmax update, PV
  auto process = [&](const uint4 (&kf)[TILES][4], const uint4 (&vf)[BS / 4], int n_valid) {
      if constexpr (MFMA) {
        float z[TILES][4];
  #pragma unroll
        for (int t = 0; t < TILES; ++t) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int m = 0; m < 4; ++m) acc = mfma16x16x32<BF16>(kf[t][m], qf[m], acc);
  #pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tok = PVM ? 8 * quad + 4 * t + v : t * 16 + quad * 4 + v;
            z[t][v] = tok < n_valid ? acc[v] * a.scale_log2 : -INFINITY;
          }
        }
        float bm = -INFINITY;
  #pragma unroll
        for (int t = 0; t < TILES; ++t)
  #pragma unroll
          for (int v = 0; v < 4; ++v) bm = fmaxf(bm, z[t][v]);
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m_run, bm);
        const float alpha = exp2f(m_run - m_new);
        float ps = 0.f;
        wave_sync_lds();
        if constexpr (PVM) {
          // P as the A operand, hi + lo halves (bf16: ~16 significant bits
          // together; fp16: scaled by 2^15 first so small weights keep their
          // bits, undone when the wave's result is written)
          uint32_t hi[8], lo[8];
  #pragma unroll
          for (int t = 0; t < TILES; ++t)
  #pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float p = exp2f(z[t][v] - m_new);
              ps += p;
              const float pa = col < G ? (BF16 ? p : p * 32768.f) : 0.f;
              const int j = 4 * t + v;
              if constexpr (BF16) {
                hi[j] = bf16_rne(pa);
                lo[j] = bf16_rne(pa - __uint_as_float(hi[j] << 16));
              } else {
                const _Float16 h16 = (_Float16)pa;
                hi[j] = __builtin_bit_cast(uint16_t, h16);
                lo[j] = __builtin_bit_cast(uint16_t, (_Float16)(pa - (float)h16));
              }
            }
          const uint4 a_hi = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16,
                                        hi[6] | hi[7] << 16);
          const uint4 a_lo = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16,
                                        lo[6] | lo[7] << 16);
          ps += __shfl_xor(ps, 16);
          ps += __shfl_xor(ps, 32);
          l_run = l_run * alpha + ps;
          m_run = m_new;
          if (quad == 0) alpha_s[wave][col] = alpha;  // every column: rows >= G stay finite
          // V tile into LDS, rows of VS elements (8-byte stores: VS*2 is 8-aligned)
  #pragma unroll
          for (int k = 0; k < BS / 4; ++k) {
            uint2* dst = reinterpret_cast<uint2*>(&v_s[wave][(quad + 4 * k) * VS + col * 8]);
            dst[0] = make_uint2(vf[k].x, vf[k].y);
            dst[1] = make_uint2(vf[k].z, vf[k].w);
          }
          wave_sync_lds();
          const float al0 = alpha_s[wave][quad * 4], al1 = alpha_s[wave][quad * 4 + 1];
          const float al2 = alpha_s[wave][quad * 4 + 2], al3 = alpha_s[wave][quad * 4 + 3];
          const uint16_t* vcol = &v_s[wave][(8 * quad) * VS + col];
  #pragma unroll
          for (int c = 0; c < 8; ++c) {
            // B operand: V[8*quad + j][c*16 + col], j = 0..7
            uint32_t b[8];
  #pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = vcol[j * VS + c * 16];
            const uint4 bv = make_uint4(b[0] | b[1] << 16, b[2] | b[3] << 16, b[4] | b[5] << 16,
                                        b[6] | b[7] << 16);
            oc[c][0] *= al0;
            oc[c][1] *= al1;
            oc[c][2] *= al2;
            oc[c][3] *= al3;
            oc[c] = mfma16x16x32<BF16>(a_hi, bv, oc[c]);
            oc[c] = mfma16x16x32<BF16>(a_lo, bv, oc[c]);
          }
        } else {
  #pragma unroll
          for (int t = 0; t < TILES; ++t)
  #pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float p = exp2f(z[t][v] - m_new);
              ps += p;
              if (col < G) p_s[wave][t * 16 + quad * 4 + v][col] = p;
            }
          ps += __shfl_xor(ps, 16);
          ps += __shfl_xor(ps, 32);
          l_run = l_run * alpha + ps;
          m_run = m_new;
          if (quad == 0 && col < G) alpha_s[wave][col] = alpha;
          wave_sync_lds();
  #pragma unroll
          for (int h = 0; h < G; ++h) {
            const float al = alpha_s[wave][h];
  #pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= al;
          }
        }
      } else {
        // z[t][h]: logit of token t*16 + col for head h, partial over the
        // lane's 32 dims, then summed across the four quads
        float z[TILES][GV];
  #pragma unroll
        for (int t = 0; t < TILES; ++t)
  #pragma unroll
          for (int h = 0; h < GV; ++h) {
            float acc = 0.f;
  #pragma unroll
            for (int m = 0; m < 4; ++m) {
              acc = dot2<BF16>(kf[t][m].x, qv[h][m].x, acc);
              acc = dot2<BF16>(kf[t][m].y, qv[h][m].y, acc);
              acc = dot2<BF16>(kf[t][m].z, qv[h][m].z, acc);
              acc = dot2<BF16>(kf[t][m].w, qv[h][m].w, acc);
            }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            z[t][h] = t * 16 + col < n_valid ? acc * a.scale_log2 : -INFINITY;
          }
        wave_sync_lds();
  #pragma unroll
        for (int h = 0; h < GV; ++h) {
          float bm = z[0][h];
  #pragma unroll
          for (int t = 1; t < TILES; ++t) bm = fmaxf(bm, z[t][h]);
          bm = row_max<16>(bm);
          const float m_new = fmaxf(mh[h], bm);
          const float alpha = exp2f(mh[h] - m_new);
          float ps = 0.f;
  #pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const float p = exp2f(z[t][h] - m_new);
            ps += p;
            if ((h & 3) == quad) p_s[wave][t * 16 + col][h] = p;
          }
          lh[h] = lh[h] * alpha + row_sum<16>(ps);
          mh[h] = m_new;
  #pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
        }
        wave_sync_lds();
      }
      if constexpr (!PVM) {
  #pragma unroll
        for (int k = 0; k < BS / 4; ++k) {
          float vv[8];
          unpack8<BF16>(vf[k], vv);
          const int t = quad + 4 * k;
  #pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = p_s[wave][t][h];
  #pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] = fmaf(p, vv[e], o[h][e]);
          }
        }
      }
  };

  {
#pragma unroll 1
    for (int k = 0; k < MAXB; ++k) {
      if (i0 + k >= i1) break;
      // block id and table entry of the wave's k-th block, from the lanes
      // that fetched them (k is uniform: a scalar lane select)
      const int blk = __builtin_amdgcn_readlane(mv, k);
      const int64_t ent = __builtin_amdgcn_readlane(mv, MAXB + k);
      const int64_t slice = a.hw ? ent : ent * a.Hkv + g;
      const uint16_t* Kp = reinterpret_cast<const uint16_t*>(a.pool + slice * a.slice_bytes);
      const int n_valid = (int)min<int64_t>(BS, (int64_t)n_tokens - (int64_t)blk * BS);
      // not a valid entry (unused, or outside the request or the pool): nothing to read
      if (ent < 0 || slice >= a.n_slices || blk < 0 || n_valid <= 0) continue;
      uint4 kf[TILES][4], vf[BS / 4];
      load_tiles(Kp, kf, vf);
      process(kf, vf, n_valid);
    }
  }

  if constexpr (PVM) {
    // the MFMA accumulators already sum every token of the wave; the o
    // partials overwrite this wave's V tile, so its last reads go first
    wave_sync_lds();
    const float osc = BF16 ? 1.f : 1.f / 32768.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (quad * 4 + i < G) wo(wave)[(quad * 4 + i) * D + c * 16 + col] = oc[c][i] * osc;
    if (quad == 0 && col < G) {
      wm[wave][col] = m_run;
      wl[wave][col] = l_run;
    }
  } else {
    // sum the four token groups of the wave
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[h][e] += __shfl_xor(o[h][e], 16);
        o[h][e] += __shfl_xor(o[h][e], 32);
      }
    if (quad == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) wo(wave)[h * D + col * 8 + e] = o[h][e];
      if constexpr (MFMA) {
        if (col < G) {
          wm[wave][col] = m_run;
          wl[wave][col] = l_run;
        }
      } else if (col == 0) {
#pragma unroll
        for (int h = 0; h < GV; ++h) {
          wm[wave][h] = mh[h];
          wl[wave][h] = lh[h];
        }
      }
    }
  }
  __syncthreads();

  // merge the waves and write one partial per (head, split)
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, j = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) M = fmaxf(M, wm[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) {
      const float f = wm[w][h] == -INFINITY ? 0.f : exp2f(wm[w][h] - M);
      L = fmaf(wl[w][h], f, L);
      O = fmaf(wo(w)[h * D + j], f, O);
    }
    float* P = a.part + (((int64_t)r * a.Hq + (int64_t)g * G + h) * a.S + s) * PART;
    if (j == 0) {
      P[0] = M;
      P[1] = L;
    }
    P[2 + j] = O;
  }

}

// One workgroup per (request, head), one thread per dim: single-pass merge
// of the request's non-empty splits in order (ceil(count / blocks per
// split) of the S), loads batched NB splits at a time.  The first batch is
// loaded together with the selection count rather than after it (split
// indices clamped to S - 1, inside the request's rows): one memory round
// trip, not two.  Splits past the count hold stale workspace bytes, which
// are read and never used.
template <int NB>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(const float* part, float* out, int S,
                                                          const int32_t* sel_cnt, int k_stride,
                                                          int per_split, int Hq) {
  const int64_t rh = blockIdx.x;  // request * Hq + head
  const int j = threadIdx.x;
  const float* P = part + rh * S * PART;
  const int cnt_raw = sel_cnt[rh / Hq];
  float m[NB], l[NB], o[NB];
  auto load = [&](int s0, int last) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int t = min(s0 + k, last);
      m[k] = P[t * PART];
      l[k] = P[t * PART + 1];
      o[k] = P[t * PART + 2 + j];
    }
  };
  float M = -INFINITY, L = 0.f, O = 0.f;
  // branch-free, so that no load waits behind a test of an earlier split
  auto merge = [&](int s0, int Sr) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const bool use = s0 + k < Sr && m[k] != -INFINITY;
      const float mk = use ? m[k] : -INFINITY;
      const float Mn = fmaxf(M, mk);
      const float fa = M == -INFINITY ? 0.f : exp2f(M - Mn);  // rescales what is merged so far
      const float fb = use ? exp2f(mk - Mn) : 0.f;           // weighs this split
      L = fmaf(L, fa, (use ? l[k] : 0.f) * fb);
      O = fmaf(O, fa, (use ? o[k] : 0.f) * fb);
      M = Mn;
    }
  };
  load(0, S - 1);
  const int cnt = min(cnt_raw, k_stride);
  const int Sr = min(S, (cnt + per_split - 1) / per_split);
  merge(0, Sr);
  for (int s0 = NB; s0 < Sr; s0 += NB) {
    load(s0, Sr - 1);
    merge(s0, Sr);
  }
  out[rh * kHeadDim + j] = L > 0.f ? O / L : 0.f;
}

// Selected blocks per wave (at most MAXB); KVOFF_ATT_BPW overrides the
// default for tuning sweeps.  Fewer, longer workgroups launch faster and
// leave fewer split partials, as long as the grid still covers the 256
// compute units.  Measured, attention / combine from clean HBM:
//   Llama-3-8B layer (G = 4, k 64): 2 blocks 29.3-29.6 us, 4 27.7-28.1,
//     8 27.1-27.4 (256 workgroups);
//   variable-recall layer (G = 8, k up to 572): 4 blocks 190 / 12.7 us,
//     8 186.5-186.9 / 10.5-10.6 us;
//   the same shapes at batch 8: 8 blocks leave 128 workgroups, 24.4-24.8
//     against 16.8 us with 4;
//   batch 1, 4K context, top-32 (latency-bound): 2 blocks 7.7 us, 4 9.9.
int attend_bpw(int32_t n_req, int32_t Hkv, int32_t k_stride, int G) {
  static const int forced = [] {
    const char* e = std::getenv("KVOFF_ATT_BPW");
    const int v = e ? std::atoi(e) : 0;
    return v >= 1 && v <= MAXB ? v : 0;
  }();
  if (forced) return forced;
  if (k_stride < 64) return G < 8 ? 2 : 4;
  const int64_t wg8 = (int64_t)n_req * Hkv * ((k_stride + ATT_WAVES * 8 - 1) / (ATT_WAVES * 8));
  return wg8 >= 256 ? 8 : 4;
}

}  // namespace

int attend_splits(int32_t n_req, int32_t Hkv, int32_t k_stride, int G) {
  const int per = ATT_WAVES * attend_bpw(n_req, Hkv, k_stride, G);
  return (k_stride + per - 1) / per;
}

size_t attend_ws_bytes(const kvoff_ctx* ctx, int32_t n_req, int32_t k_stride) {
  return (size_t)n_req * ctx->cfg.num_q_heads *
         attend_splits(n_req, ctx->cfg.num_kv_heads, k_stride, ctx->G) * PART * sizeof(float);
}

namespace {

template <int G, int BS, bool MFMA>
void launch_g_bs_qk(const AttendArgs& a, bool bf16, dim3 grid, hipStream_t s, KEv ev) {
  if (bf16)
    KVOFF_LAUNCH(ev, (attend_kernel<G, BS, true, MFMA>), grid, dim3(256), 0, s, a);
  else
    KVOFF_LAUNCH(ev, (attend_kernel<G, BS, false, MFMA>), grid, dim3(256), 0, s, a);
}

template <int G, int BS>
void launch_g_bs(const AttendArgs& a, bool bf16, bool mfma, dim3 grid, hipStream_t s, KEv ev) {
  if constexpr (G <= 8) {  // kvoff_set_attention_qk admits VALU only for G <= 8
    if (!mfma) return launch_g_bs_qk<G, BS, false>(a, bf16, grid, s, ev);
  }
  launch_g_bs_qk<G, BS, true>(a, bf16, grid, s, ev);
}

template <int G>
void launch_g(const AttendArgs& a, int bs, bool bf16, bool mfma, dim3 grid, hipStream_t s, KEv ev) {
  if (bs == 16)
    launch_g_bs<G, 16>(a, bf16, mfma, grid, s, ev);
  else
    launch_g_bs<G, 32>(a, bf16, mfma, grid, s, ev);
}

}  // namespace

int launch_attend(const kvoff_ctx* ctx, const BatchIds& b, int32_t mode, const void* q_dev,
                  const void* pool, int64_t n_slots, const int32_t* table, const int32_t* sel_idx,
                  const int32_t* sel_cnt, int32_t k_stride, float scale, float* out, void* ws,
                  hipStream_t stream) {
  AttendArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.q = (const uint16_t*)q_dev;
  a.pool = (const uint8_t*)pool;
  a.table = table;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.part = (float*)ws;
  a.slice_bytes = ctx->slice_bytes;
  a.n_slices = n_slots * ctx->cfg.num_kv_heads;
  a.k_stride = k_stride;
  a.bpw = attend_bpw(b.n, ctx->cfg.num_kv_heads, k_stride, ctx->G);
  a.S = attend_splits(b.n, ctx->cfg.num_kv_heads, k_stride, ctx->G);
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.hw = mode == KVOFF_HEADWISE;
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)a.S, (unsigned)a.Hkv, (unsigned)b.n);
  const bool bf16 = ctx->cfg.dtype == KVOFF_BF16;
  const int bs = ctx->cfg.block_size;
  const bool mfma = ctx->attn_qk == KVOFF_QK_MFMA;
  const KEv ev = kernel_events(ctx, KT_ATTEND);
  switch (ctx->G) {
    case 1: launch_g<1>(a, bs, bf16, mfma, grid, stream, ev); break;
    case 2: launch_g<2>(a, bs, bf16, mfma, grid, stream, ev); break;
    case 4: launch_g<4>(a, bs, bf16, mfma, grid, stream, ev); break;
    case 8: launch_g<8>(a, bs, bf16, mfma, grid, stream, ev); break;
    default: launch_g<16>(a, bs, bf16, mfma, grid, stream, ev); break;
  }
  KVOFF_HIP(hipGetLastError());
  const KEv ev_c = kernel_events(ctx, KT_COMBINE);
  // splits merged per batch of loads: up to 32, so that a long selection
  // (36 splits at the variable-recall layer) waits for two rounds of loads
  // instead of five (combine 16.0 -> 12.9 us there); no more than S needs
  const int nb = a.S > 16 ? 32 : a.S > 8 ? 16 : 8;
  if (nb == 32)
    KVOFF_LAUNCH(ev_c, combine_kernel<32>, dim3((unsigned)(b.n * a.Hq)), dim3(kHeadDim), 0, stream,
                 (const float*)a.part, out, (int)a.S, sel_cnt, (int)k_stride, ATT_WAVES * a.bpw, (int)a.Hq);
  else if (nb == 16)
    KVOFF_LAUNCH(ev_c, combine_kernel<16>, dim3((unsigned)(b.n * a.Hq)), dim3(kHeadDim), 0, stream,
                 (const float*)a.part, out, (int)a.S, sel_cnt, (int)k_stride, ATT_WAVES * a.bpw, (int)a.Hq);
  else
    KVOFF_LAUNCH(ev_c, combine_kernel<8>, dim3((unsigned)(b.n * a.Hq)), dim3(kHeadDim), 0, stream,
                 (const float*)a.part, out, (int)a.S, sel_cnt, (int)k_stride, ATT_WAVES * a.bpw, (int)a.Hq);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
