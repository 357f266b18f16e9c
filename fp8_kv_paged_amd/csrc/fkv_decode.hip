// Split-KV combine: merges the fp32 partials (m, l, O) that the decode kernels write when a
// (sequence, KV head) is cut into several splits and the splits are not merged inside the
// decode kernel itself (the row-group kernel always; the 32-row kernel when its grid does not
// fit on the chip at once, and for long query windows). Also the launch dispatcher of the
// decode kernels.
//
// Operation: the split-KV reduction of exact paged attention, with a fixed, deterministic
// order ("Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70", section "Promotion gates": a
// second fresh start must reproduce the result).
#include "fkv_device.h"
#include "fkv_internal.h"

namespace fkv {

// Merges the split partials of each (sequence, KV head) row in split order:
// out = v_scale * sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// A thread owns 4 dimensions of one row; a group of 128 threads holds 4 rows. Splits are
// folded 8 at a time, in split order, into a running maximum, row sum and output (the same
// order for every call); the (m, l) and output pieces of 32 splits are requested before any
// is used (one memory round trip per 32 splits).
constexpr int kCombineRows = 4;
constexpr int kCombineChunk = 8;
constexpr int kCombineAhead = 4;  // chunks whose loads are in flight together

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a, int kfp8) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = a.group, M = a.q_len, GM = G * M;
  const int wl = a.window_left;
  int L = a.seq_lens[b];
  L = min(L, min(a.max_seq_len, a.max_blocks * a.block_size));
  const int lo_u = (wl < 0) ? 0 : max(0, L - M - wl);
  const int t_first = lo_u / kTile;
  const int t_end = L > 0 ? (L + kTile - 1) / kTile : 0;
  const int ntiles = max(0, t_end - t_first);
  const int nsplit = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (nsplit <= 1) return;
  const int r = blockIdx.x * kCombineRows + (threadIdx.x >> 5);
  const int d4 = threadIdx.x & 31;
  if (r >= GM) return;
  const int64_t base = ((int64_t)b * a.num_kv_heads + g) * a.max_splits;
  const int64_t ml_stride = 2 * (int64_t)a.rows_pad;
  const int64_t o_stride = (int64_t)a.rows_pad * kHeadDim;
  const float* mlp = a.ws_ml + base * ml_stride + r;
  const float* op = a.ws_o + (base * a.rows_pad + r) * kHeadDim + 4 * d4;

  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t acc{0.f, 0.f, 0.f, 0.f};
  // kCombineAhead chunks are requested together (one round trip for up to 32 splits), then
  // folded one chunk at a time as their loads return
  for (int g0 = 0; g0 < nsplit; g0 += kCombineAhead * kCombineChunk) {
    float ms[kCombineAhead][kCombineChunk], ls[kCombineAhead][kCombineChunk];
    f32x4_t os[kCombineAhead][kCombineChunk];
#pragma unroll
    for (int c = 0; c < kCombineAhead; ++c) {
      if (g0 + c * kCombineChunk >= nsplit) break;  // chunks past the last split are not requested
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        const int sj = min(g0 + c * kCombineChunk + j, nsplit - 1);  // clamped: in-range loads, unused past the end
        ms[c][j] = mlp[sj * ml_stride];
        ls[c][j] = mlp[sj * ml_stride + a.rows_pad];
        os[c][j] = *reinterpret_cast<const f32x4_t*>(op + sj * o_stride);
      }
    }
#pragma unroll
    for (int c = 0; c < kCombineAhead; ++c) {
      const int s0 = g0 + c * kCombineChunk;
      if (s0 >= nsplit) break;
      float mc = mrun;
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j)
        if (s0 + j < nsplit) mc = fmaxf(mc, ms[c][j]);
      // rescale what has been folded so far to the new maximum, then fold this chunk in order
      const float keep = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mc);
      lrun *= keep;
      acc *= keep;
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        if (s0 + j < nsplit) {
          const float wgt = (ms[c][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[c][j] - mc);
          lrun += wgt * ls[c][j];
          acc += os[c][j] * wgt;
        }
      }
      mrun = mc;
    }
  }
  const float vsc = kfp8 ? *a.v_scale : 1.0f;
  const float mul = lrun > 0.f ? vsc / lrun : 0.f;
  const int i = r / G, h = g * G + (r - i * G);
  store_out4(a.out, a.out_bf16, (((int64_t)b * M + i) * a.num_q_heads + h) * kHeadDim + 4 * d4, acc * mul);
}

hipError_t launch_combine(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  const int rows = a.group * a.q_len;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((rows + kCombineRows - 1) / kCombineRows, a.num_kv_heads, a.num_seqs),
                     dim3(32 * kCombineRows), 0, stream, a, fp8 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const SplitShapeInfo& shape, bool fp8, hipStream_t stream,
                         bool* launched_combine) {
  *launched_combine = false;
  if (a.num_seqs == 0) return hipSuccess;
  hipError_t e;
  if (shape.groups_per_cu == 0) {
    e = launch_rows(a, shape.ntw, fp8, stream);
  } else {
    // row tiles per work group (rows_pad / 32 row tiles in row_groups groups); layout 6 holds
    // two row tiles per wave
    e = launch_m32(a, a.rows_pad / 32 / a.row_groups, shape.groups_per_cu == -3 ? 2 : 1, a.key_lanes, fp8, stream);
  }
  if (e != hipSuccess) return e;
  if (a.max_splits > 1 && !a.fused_combine) {
    e = launch_combine(a, fp8, stream);
    *launched_combine = true;
  }
  return e;
}

}  // namespace fkv
