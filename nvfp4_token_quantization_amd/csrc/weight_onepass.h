// weight_onepass.h -- the NVFP4 weight quantizer in one HBM pass (gfx950).
//
// Method: the Miles page ("Towards Blackwell-Native 8-bit and 4-bit RL"),
// section 并行度与张量转换的一致性契约 (one FP32 outer scale per tensor or per
// expert, S = amax(W_g) / 2688, a fused gate|up expert weight sharing one)
// and section 速读 (block scales and codes exactly as for activation rows).
//
// Every element of a group is encoded with the group's amax, so the amax must
// be complete before the first element is encoded.  The two-pass form reads
// the weight twice (amax pass, encode pass).  Here each group is read once and
// held in registers by a team of workgroups until the team agrees on its amax:
//  - one 1024-thread workgroup per CU (its registers allow no second one, so
//    all are resident together); workgroup b is member b / T of team b % T.
//    Workgroups are dealt round-robin to the 8 XCDs, so when T is a multiple
//    of 8 a team's members share one XCD;
//  - team t quantizes groups t, t + T, t + 2T, ...  Per round each wave
//    holds its rows of the group in registers (the row layout of the row
//    kernels: L lanes per row, U 16-byte half-blocks per lane, up to NG row
//    groups);
//  - the team meets once per round.  All but its last round meet through
//    slots: the first 64 code dwords of the team's next group, zeroed by a
//    fill kernel before the launch.  A member stores its workgroup's maximum
//    (bf16 magnitude bits, with a valid bit) in its slot, and one wave reads
//    every member's slot in one load per poll until all are valid, then
//    takes their maximum (order-free, so deterministic).  No member writes
//    those dwords while encoding; the team's last member to leave its last
//    round writes them, once no member can still be reading a slot;
//  - the last round meets through amax_out[g] and s[g] (also zeroed): an
//    atomic max of the workgroup's maximum on amax_out[g] and, once that
//    atomic has returned, an atomic add to the low 16 bits of s[g]; a member
//    waits until every member has counted in and then reads amax_out[g]; the
//    high 16 bits of s[g] count the members out and the last to leave
//    stores S over the counter (and writes the slot areas);
//  - as each row group is encoded its registers receive the member's rows of
//    the team's next group, so the weight stream continues through the
//    encode and the wait;
//  - the wait is bounded in time: a member that gives up derives the group
//    amax by reading the whole group itself (the same maximum, hence the same
//    bits) and goes on, so every wave ends whatever else runs on the device.
#pragma once

#include "quant_rows.h"

namespace nvfp4 {

constexpr int OP_WAVES = 16;  // waves per workgroup (four per SIMD, up to 128 VGPRs each)
// the library's settings: groups of at least 512 KiB of bf16 (smaller ones
// gain little over the two passes); at least 8 teams, so that every team
// lies on one XCD (a wait on members in other XCDs sees their counts late:
// measured several times slower); a 10 ms bound on a member's wait
constexpr int64_t OP_MIN_GROUP_BYTES = (int64_t)512 << 10;
constexpr int OP_MIN_TEAMS = 8;
constexpr double OP_LIMIT_MS = 10.0;
// slot rounds: the slots are the first OP_SLOTS code dwords of the team's
// next group (512 elements), and each workgroup keeps the amax of up to
// OP_MAX_ROUNDS rounds to write those dwords at the end
constexpr int OP_SLOTS = 64;
constexpr int OP_MAX_ROUNDS = 1024;
// row groups a wave holds: at most 8, and at most 12 uint4 per lane (48
// VGPRs of bf16; the encode needs the rest of the 128)
template <int U>
constexpr int op_ngmax() { return U >= 12 ? 1 : (12 / U < 8 ? 12 / U : 8); }

// Thread 0 of a member: count in for group g with this workgroup's maximum
// (bf16 magnitude bits << 16): an atomic max on amax_out[g], then, once that
// atomic has returned, the count in the low 16 bits of s[g].  A member that
// sees every arrival counted therefore also sees every maximum applied.
__device__ __forceinline__ void op_arrive(uint32_t* amax_bits, uint32_t* cnt, uint32_t mine) {
  const uint32_t prev = __hip_atomic_fetch_max(amax_bits, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t one = 1u;
  asm volatile("" : "+v"(one) : "v"(prev));  // the add waits for the max's reply
  __hip_atomic_fetch_add(cnt, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: wait until `members` have counted in, then read the group amax
// bits.  ok = false, and 0, when the time limit (wall-clock ticks) runs out
// first.
__device__ __forceinline__ uint32_t op_wait(uint32_t* amax_bits, uint32_t* cnt, uint32_t members,
                                            uint64_t limit, bool& ok) {
  const uint64_t t0 = wall_clock64();
  while ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFFu) < members) {
    if (wall_clock64() - t0 >= limit) {
      ok = false;
      return 0u;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  ok = true;
  return __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: count out of group g in the high 16 bits of s[g]; the last
// member to leave (every member has counted in and finished waiting) stores
// S over the counter.
__device__ __forceinline__ bool op_depart(float* s, int g, uint32_t members, float A) {
  uint32_t* c = reinterpret_cast<uint32_t*>(s) + g;
  const uint32_t old = __hip_atomic_fetch_add(c, 0x10000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old >> 16) != members - 1) return false;
  __hip_atomic_store(c, __float_as_uint(row_scale(A).S), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Wave 0 of a member, slot round: post this workgroup's maximum (bf16
// magnitude bits) with a valid bit in its slot, then read every member's
// slot in one load per poll until all are valid.  Returns the group amax as
// fp32 bits; ok = false, and 0, when the time limit runs out first.
__device__ __forceinline__ uint32_t op_slot_wait(uint32_t* slots, uint32_t member, uint32_t members,
                                                 uint32_t mine, uint64_t limit, bool& ok) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) __hip_atomic_store(slots + member, 0x10000u | mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint32_t v = (uint32_t)lane < members
                           ? __hip_atomic_load(slots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0x10000u;
    if (__all((v & 0x10000u) != 0u)) {
      ok = true;
      return group_max_u32<64>(v & 0xFFFFu) << 16;
    }
    if (wall_clock64() - t0 >= limit) {
      ok = false;
      return 0u;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The whole workgroup: amax bits (<< 16) of one group's `elems` bf16 values,
// read from HBM (the path of a member whose wait ran out).
__device__ __forceinline__ uint32_t op_group_amax(const uint16_t* __restrict__ wg, int64_t elems,
                                                  uint32_t* red) {
  const uint4* v = reinterpret_cast<const uint4*>(wg);
  const int64_t nv = elems / 8;
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < nv; i += 64 * OP_WAVES) m = max(m, half_amax_bits(ld_stream(v + i)));
  m = group_max_u32<64>(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t b = 0;
#pragma unroll
  for (int w = 0; w < OP_WAVES; ++w) b = max(b, red[w]);
  __syncthreads();
  return b << 16;
}

struct OpArgs {
  const uint16_t* w;
  int groups;
  int64_t R, k;
  int nh, teams, ng;
  int slots;  // 1: slot rounds (all but each team's last), 0: every round by atomics
  uint64_t limit;
  float* amax;
  uint8_t* q;
  uint8_t* sb;
  float* s;
};

// Lane state: row of row group i held by this lane = lr0 + i * lstep (within
// its group); lane j of its row; the workgroup's index in its team and the
// team's size.
struct OpLane {
  int64_t lr0, lstep;
  int j;
  uint32_t member, members;
};

template <int L, int U>
__device__ __forceinline__ void op_load(RowData<U> (&r)[op_ngmax<U>()], const OpArgs& a, const OpLane& l,
                                        int g) {
#pragma unroll
  for (int i = 0; i < op_ngmax<U>(); ++i)
    if (i < a.ng)
      load_rows<L, U, MODE_ROW>(a.w, (int64_t)(g + 1) * a.R, a.k, a.nh, (int64_t)g * a.R + l.lr0 + i * l.lstep,
                                l.j, nullptr, a.R, r[i]);
}

// The team's last member out of its last round: the first OP_SLOTS code
// dwords of the team's groups 1.. (the slot areas, left unwritten by their
// owners) from the groups' first 512 elements and the amax of each round
// (all threads; wave w takes rounds 1 + w, 1 + w + OP_WAVES, ...).
template <int U>
__device__ __forceinline__ void op_write_slot_codes(const OpArgs& a, int team, int last_round,
                                                    const float* s_amax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int jr = 1 + wave; jr <= last_round; jr += OP_WAVES) {  // wave-uniform
    const int64_t g = team + (int64_t)jr * a.teams;
    // half-block `lane` of the group (rows are whole pairs of half-blocks,
    // so lanes 2m and 2m + 1 hold one block)
    const uint4 d = ld_stream(reinterpret_cast<const uint4*>(a.w + g * a.R * a.k) + lane);
    uint32_t code;
    float inv;
    block_scale(max(half_amax_bits(d), dpp_mov<0xB1>(half_amax_bits(d))), row_scale(s_amax[jr]), code, inv);
    reinterpret_cast<uint32_t*>(a.q + g * a.R * (a.k / 2))[lane] = encode_half(d, inv);
  }
}

// One round (all threads): the registers hold this member's rows of group g
// (the team's round jr).  Count in with the workgroup's maximum, wait for
// the team (or its time limit), encode the rows and refill the registers
// with the member's rows of group g + T as each row group is encoded, count
// out.  Slot rounds meet through slots in group g + T's codes; the team's
// last round (and every round without slots) through amax_out[g] and s[g].
template <int L, int U>
__device__ __forceinline__ void op_round(RowData<U> (&r)[op_ngmax<U>()], const OpArgs& a, const OpLane& l,
                                         int g, int jr, uint32_t* red, uint32_t* bc, float* s_amax) {
  const int gn = g + a.teams;
  const bool slotted = a.slots && gn < a.groups;  // workgroup-uniform
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < op_ngmax<U>(); ++i)
    if (i < a.ng) {
#pragma unroll
      for (int u = 0; u < U; ++u) m = max(m, half_amax_bits(r[i].d[u]));
    }
  m = group_max_u32<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (slotted) {
    if (threadIdx.x < 64) {
      uint32_t bm = 0;
#pragma unroll
      for (int v = 0; v < OP_WAVES; ++v) bm = max(bm, red[v]);
      bool ok;
      const uint32_t v = op_slot_wait(reinterpret_cast<uint32_t*>(a.q + (int64_t)gn * a.R * (a.k / 2)), l.member,
                                      l.members, bm, a.limit, ok);
      if (threadIdx.x == 0) {
        bc[0] = v;
        bc[1] = ok ? 1u : 0u;
      }
    }
  } else if (threadIdx.x == 0) {
    uint32_t bm = 0;
#pragma unroll
    for (int v = 0; v < OP_WAVES; ++v) bm = max(bm, red[v]);
    uint32_t* ab = reinterpret_cast<uint32_t*>(a.amax) + g;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(a.s) + g;
    op_arrive(ab, cnt, bm << 16);
    bool ok;
    bc[0] = op_wait(ab, cnt, l.members, a.limit, ok);
    bc[1] = ok ? 1u : 0u;
  }
  __syncthreads();
  uint32_t abits = bc[0];
  if (bc[1] == 0u) abits = op_group_amax(a.w + (int64_t)g * a.R * a.k, a.R * a.k, red);  // uniform
  const float A = __uint_as_float(abits);
  if (a.slots && threadIdx.x == 0) s_amax[jr] = A;
  __syncthreads();  // bc and red are rewritten below and by the next round
  // a slot area (the codes' first OP_SLOTS dwords of the team's groups 1..)
  // is written at the end, when no member can still be reading it
  const bool skip_slots = a.slots && jr > 0;
#pragma unroll
  for (int i = 0; i < op_ngmax<U>(); ++i)
    if (i < a.ng) {
      const int64_t lr = l.lr0 + i * l.lstep;
      const int qskip = (skip_slots && lr < OP_SLOTS) ? OP_SLOTS - (int)lr * a.nh : 0;
      r[i].amax = A;
      encode_rows<L, U, MODE_GROUP>(r[i], (int64_t)(g + 1) * a.R, a.k, a.nh, (int64_t)g * a.R + lr, l.j,
                                    nullptr, a.R, a.q, a.sb, nullptr, qskip);
      if (gn < a.groups)
        load_rows<L, U, MODE_ROW>(a.w, (int64_t)(gn + 1) * a.R, a.k, a.nh, (int64_t)gn * a.R + lr, l.j,
                                  nullptr, a.R, r[i]);
    }
  if (slotted) {
    if (threadIdx.x == 0 && l.member == 0) {
      a.amax[g] = A;
      a.s[g] = row_scale(A).S;
    }
  } else if (threadIdx.x == 0) {
    bc[2] = op_depart(a.s, g, l.members, A) ? 1u : 0u;
  }
}

// groups of R rows of k bf16 each (nh = k / 8 half-blocks per row); `teams`
// teams; each wave holds ng <= op_ngmax<U>() row groups.  amax and s, and
// with slots the first OP_SLOTS code dwords of every group, are zero on
// entry.
template <int L, int U>
__global__ __launch_bounds__(64 * OP_WAVES) void quantize_weight_onepass_kernel(OpArgs a) {
  constexpr int RPW = 64 / L, NG = op_ngmax<U>();
  __shared__ uint32_t red[OP_WAVES];
  __shared__ uint32_t bc[3];
  __shared__ float s_amax[OP_MAX_ROUNDS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int team = (int)(blockIdx.x % (unsigned)a.teams);
  OpLane l;
  l.members = (gridDim.x - (unsigned)team + (unsigned)a.teams - 1) / (unsigned)a.teams;
  l.member = blockIdx.x / (unsigned)a.teams;
  l.j = lane % L;
  // this wave's index in its team, and the team's wave count
  const int64_t wt = (int64_t)l.member * OP_WAVES + wave;
  l.lr0 = wt * RPW + lane / L;
  l.lstep = (int64_t)l.members * OP_WAVES * RPW;
  RowData<U> r[NG];
  const int g0 = team;
  if (g0 >= a.groups) return;  // workgroup-uniform
  op_load<L, U>(r, a, l, g0);
  int jr = 0;
  for (int g = g0; g < a.groups; g += a.teams, ++jr)  // workgroup-uniform
    op_round<L, U>(r, a, l, g, jr, red, bc, s_amax);
  // the team's last round met by atomics; its last member out writes the
  // slot areas of the team's groups 1 .. jr - 1
  if (a.slots) {
    __syncthreads();
    if (bc[2]) op_write_slot_codes<U>(a, team, jr - 1, s_amax);  // workgroup-uniform
  }
}

__global__ __launch_bounds__(256) void fill_zero2_kernel(float* __restrict__ a, float* __restrict__ b,
                                                         int64_t n, uint8_t* __restrict__ q, int64_t qstride) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    a[i] = 0.0f;
    b[i] = 0.0f;
  }
  if (q)  // the slot areas
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n * OP_SLOTS; i += (int64_t)gridDim.x * 256)
      reinterpret_cast<uint32_t*>(q + (i / OP_SLOTS) * qstride)[i % OP_SLOTS] = 0u;
}
typedef void (*OnePassKernel)(OpArgs);

template <int L>
static OnePassKernel op_kernel_for(int u) {
  switch (u) {
    case 1: return quantize_weight_onepass_kernel<L, 1>;
    case 2: return quantize_weight_onepass_kernel<L, 2>;
    case 3: return quantize_weight_onepass_kernel<L, 3>;
    case 4: return quantize_weight_onepass_kernel<L, 4>;
    case 5: return quantize_weight_onepass_kernel<L, 5>;
    case 6: return quantize_weight_onepass_kernel<L, 6>;
    case 7:
    case 8: return quantize_weight_onepass_kernel<L, 8>;
    default: return nullptr;
  }
}

// Lanes per row (the widest of 64, 32, 16 that divides the row's half-blocks
// into at most 8 per lane, else the narrowest that holds the row); null when
// a row needs more than 8 half-blocks per lane.
static OnePassKernel op_pick(int nh, int& lanes, int& ngmax) {
  static const int ngm[9] = {0, op_ngmax<1>(), op_ngmax<2>(), op_ngmax<3>(), op_ngmax<4>(),
                             op_ngmax<5>(), op_ngmax<6>(), op_ngmax<8>(), op_ngmax<8>()};
  int L = 0;
  if (nh % 64 == 0 && nh / 64 <= 8) L = 64;
  else if (nh % 32 == 0 && nh / 32 <= 8) L = 32;
  else if (nh % 16 == 0 && nh / 16 <= 8) L = 16;
  else if (nh <= 16 * 8) L = 16;
  else if (nh <= 32 * 8) L = 32;
  else if (nh <= 64 * 8) L = 64;
  if (!L) return nullptr;
  const int u = (nh + L - 1) / L;
  lanes = L;
  ngmax = ngm[u];
  return L == 64 ? op_kernel_for<64>(u) : L == 32 ? op_kernel_for<32>(u) : op_kernel_for<16>(u);
}

// Launches the one-pass quantizer when the shape suits it (a group of at
// least `min_group_bytes` of bf16 that a team holds in registers, with at
// least `min_teams` teams) and returns true; false leaves the call to the
// two-pass form.  `limit_ms` bounds each member's wait.
static bool launch_weight_onepass(const uint16_t* w, int64_t groups, int64_t R, int64_t k, float* amax_out,
                                  uint8_t* q, uint8_t* sb, float* s, double limit_ms,
                                  int64_t min_group_bytes, int min_teams, hipStream_t stream) {
  if (groups < 1 || R < 1 || k < 16 || groups >= ((int64_t)1 << 31)) return false;
  if (R > (((int64_t)1 << 40) / k)) return false;  // a group's bytes stay far from overflow
  if (R * k * 2 < min_group_bytes) return false;
  // the counter lives in s and the maximum in amax_out: they must be distinct
  if (amax_out + groups > s && s + groups > amax_out) return false;
  const int nh = (int)(k / 8);
  int lanes = 0, ngmax = 0;
  OnePassKernel kern = op_pick(nh, lanes, ngmax);
  if (!kern) return false;
  const int cus = nvfp4host::num_cus();
  const int64_t rgn = (R + 64 / lanes - 1) / (64 / lanes);  // row groups per group
  int teams = 0, ng = 0;
  // the most teams (fewest rounds) whose smallest team still holds a group,
  // at least min_teams of them
  for (int t = 32; t >= min_teams && t >= 1; t /= 2) {
    if (t > 1 && (t > groups || t > cus)) continue;
    const int64_t waves = (int64_t)(cus / t) * OP_WAVES;
    const int64_t need = (rgn + waves - 1) / waves;
    if (need <= ngmax) {
      teams = t;
      ng = (int)need;
      break;
    }
  }
  if (!teams || cus >= 65536) return false;
  const double ticks = limit_ms * (double)nvfp4host::wall_clock_khz();
  const uint64_t limit = ticks <= 0.0 ? 0 : (uint64_t)ticks;
  // slot rounds when one wave can read every member's slot, a group's codes
  // hold the slot area, and each workgroup can keep every round's amax
  const int64_t members = (cus + teams - 1) / teams;
  const int64_t rounds = (groups + teams - 1) / teams;
  const int slots = (members <= 64 && R * (k / 2) >= 4 * OP_SLOTS && rounds <= OP_MAX_ROUNDS) ? 1 : 0;
  const unsigned gz = (unsigned)((groups * (slots ? OP_SLOTS : 1) + 255) / 256);
  hipLaunchKernelGGL(fill_zero2_kernel, dim3(gz < 1024 ? gz : 1024), dim3(256), 0, stream, amax_out, s, groups,
                     slots ? q : nullptr, R * (k / 2));
  OpArgs a;
  a.slots = slots;
  a.w = w;
  a.groups = (int)groups;
  a.R = R;
  a.k = k;
  a.nh = nh;
  a.teams = teams;
  a.ng = ng;
  a.limit = limit;
  a.amax = amax_out;
  a.q = q;
  a.sb = sb;
  a.s = s;
  hipLaunchKernelGGL(kern, dim3((unsigned)cus), dim3(64 * OP_WAVES), 0, stream, a);
  return true;
}

}  // namespace nvfp4
