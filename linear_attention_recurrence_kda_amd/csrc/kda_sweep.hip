// Decode step and verify-and-replay: a bandwidth-bound sweep over per-head
// fp32 states.
//
// One workgroup owns one (session, head) state S (DK x DV, fp32) for the whole
// call and keeps it in registers: thread t holds float4 column group
// cg = t % CG (CG = DV / 4) of rows rg, rg + RG, ... (RG = NT / CG), so one
// wave reads whole 16-byte-aligned rows and every state byte is loaded once
// and stored once per call, fully coalesced.
//
// Each step follows the recurrence of the "Serve 模块交互式演示" page (§1.3
// kda_step) with the decay applied before the error, as the "Kimi Linear 的
// KDA 缓存" page (section "KDA 的递推与充分状态") orders it:
//   e_i = exp(a_i);  p_j = sum_i e_i k_i S_ij;  r_j = sum_i e_i q_i S_ij
//   d_j = v_j - p_j;  S_ij <- e_i S_ij + beta k_i d_j
//   o_j = r_j + beta d_j (k . q)          (= S_new^T q)
// The sums over i (the key dimension) are split over row groups: partial sums
// in registers, a cross-lane butterfly inside the wave, then LDS across
// waves.  Replay (the "verify_and_replay" of §1.2) runs n_accepted such steps
// on the register-resident state, reading a committed state it never writes.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

template <int DK, int DV>
struct SweepShape {
  static constexpr int CG = DV / 4;                       // float4 column groups
  static constexpr int NT = (CG * DK < 256) ? CG * DK : 256;  // threads
  static constexpr int RG = NT / CG;                      // row groups
  static constexpr int RPT = DK / RG;                     // rows per thread
  static constexpr int NW = NT / kWave;                   // waves (>= 1)
  static_assert(DV % 4 == 0 && NT % kWave == 0 && DK % RG == 0, "shape");
};

template <int DK, int DV, typename InT>
__global__ __launch_bounds__((SweepShape<DK, DV>::NT)) void sweep_kernel(
    const float* s_in, float* s_out, const InT* __restrict__ q, const InT* __restrict__ k,
    const InT* __restrict__ v, const InT* __restrict__ a, const InT* __restrict__ beta,
    const int32_t* __restrict__ n_accepted, int t_draft, int B, int H, InT* __restrict__ o,
    int o_steps, int32_t* __restrict__ err_flag) {
  using Sh = SweepShape<DK, DV>;
  constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NW = Sh::NW, NT = Sh::NT;

  const int bh = blockIdx.x;  // b * H + h
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  __shared__ float s_k[DK], s_q[DK], s_e[DK], s_v[DV];
  __shared__ float s_beta;
  __shared__ float s_red[NW > 1 ? NW : 1][CG][9];

  int n = t_draft;
  if (n_accepted != nullptr) {
    n = n_accepted[b];
    if (n < 0 || n > t_draft) {
      if (err_flag != nullptr && tid == 0) *err_flag = 1;
      n = n < 0 ? 0 : t_draft;
    }
  }

  // Load the state once.
  const size_t sbase = static_cast<size_t>(bh) * DK * DV;
  float4 S[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + m * RG;
    S[m] = *reinterpret_cast<const float4*>(s_in + sbase + static_cast<size_t>(r) * DV + 4 * cg);
  }

  for (int i = 0; i < n; ++i) {
    const size_t tok = static_cast<size_t>(i) * B * H + bh;  // (i, b, h) in (Td, B, H)
    __syncthreads();  // previous step's readers of the LDS inputs are done
    for (int x = tid; x < DK; x += NT) {
      s_k[x] = to_f32(k[tok * DK + x]);
      s_q[x] = to_f32(q[tok * DK + x]);
      s_e[x] = fast_exp(to_f32(a[tok * DK + x]));
    }
    for (int x = tid; x < DV; x += NT) s_v[x] = to_f32(v[tok * DV + x]);
    if (tid == 0) s_beta = to_f32(beta[tok]);
    __syncthreads();

    // Partial sums over this thread's rows.
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      const float e = s_e[r], kr = s_k[r] * e, qr = s_q[r] * e;
      kq += s_k[r] * s_q[r];
      pk[0] += kr * S[m].x; pk[1] += kr * S[m].y; pk[2] += kr * S[m].z; pk[3] += kr * S[m].w;
      pq[0] += qr * S[m].x; pq[1] += qr * S[m].y; pq[2] += qr * S[m].z; pq[3] += qr * S[m].w;
    }
    // Butterfly over the row groups that share a wave (lanes cg, cg+CG, ...).
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] += __shfl_xor(pk[c], off);
        pq[c] += __shfl_xor(pq[c], off);
      }
      kq += __shfl_xor(kq, off);
    }
    if constexpr (NW > 1) {
      if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s_red[wave][lane][c] = pk[c];
          s_red[wave][lane][4 + c] = pq[c];
        }
        s_red[wave][lane][8] = kq;
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 4; ++c) { pk[c] = 0.f; pq[c] = 0.f; }
      kq = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pk[c] += s_red[w][cg][c];
          pq[c] += s_red[w][cg][4 + c];
        }
        kq += s_red[w][cg][8];
      }
    }

    const float bt = s_beta;
    float d[4], out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d[c] = s_v[4 * cg + c] - pk[c];
      out[c] = pq[c] + bt * d[c] * kq;
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      const float e = s_e[r], bk = bt * s_k[r];
      S[m].x = e * S[m].x + bk * d[0];
      S[m].y = e * S[m].y + bk * d[1];
      S[m].z = e * S[m].z + bk * d[2];
      S[m].w = e * S[m].w + bk * d[3];
    }
    if (rg == 0) {
      InT* op = o + (static_cast<size_t>(bh) * o_steps + i) * DV + 4 * cg;
#pragma unroll
      for (int c = 0; c < 4; ++c) op[c] = from_f32<InT>(out[c]);
    }
  }

  // Rows past the accepted prefix are zero.
  if (rg == 0) {
    for (int i = n; i < o_steps; ++i) {
      InT* op = o + (static_cast<size_t>(bh) * o_steps + i) * DV + 4 * cg;
#pragma unroll
      for (int c = 0; c < 4; ++c) op[c] = from_f32<InT>(0.f);
    }
  }

#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + m * RG;
    *reinterpret_cast<float4*>(s_out + sbase + static_cast<size_t>(r) * DV + 4 * cg) = S[m];
  }
}

template <int DK, int DV, typename InT>
hipError_t launch_sweep_t(const SweepArgs& p) {
  using Sh = SweepShape<DK, DV>;
  const dim3 grid(static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H));
  hipLaunchKernelGGL((sweep_kernel<DK, DV, InT>), grid, dim3(Sh::NT), 0, p.stream, p.s_in,
                     p.s_out, static_cast<const InT*>(p.q), static_cast<const InT*>(p.k),
                     static_cast<const InT*>(p.v), static_cast<const InT*>(p.a),
                     static_cast<const InT*>(p.beta), p.n_accepted, p.t_draft, p.B, p.H,
                     static_cast<InT*>(p.o), p.o_steps, p.err_flag);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_sweep_dt(const SweepArgs& p) {
  return p.bf16 ? launch_sweep_t<DK, DV, bf16raw>(p) : launch_sweep_t<DK, DV, float>(p);
}

template <int DK>
hipError_t launch_sweep_dv(const SweepArgs& p) {
  switch (p.dv) {
    case 16: return launch_sweep_dt<DK, 16>(p);
    case 32: return launch_sweep_dt<DK, 32>(p);
    case 64: return launch_sweep_dt<DK, 64>(p);
    case 128: return launch_sweep_dt<DK, 128>(p);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sweep(const SweepArgs& p) {
  switch (p.dk) {
    case 16: return launch_sweep_dv<16>(p);
    case 32: return launch_sweep_dv<32>(p);
    case 64: return launch_sweep_dv<64>(p);
    case 128: return launch_sweep_dv<128>(p);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
