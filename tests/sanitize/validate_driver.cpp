// Drives every host-side argument check of the C ABI (csrc/validate.cpp)
// over a grid of valid, invalid and extreme arguments (negative sizes,
// INT64 limits, size products that overflow, overlapping and null
// pointers), so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer sees every path.  Pointers are never
// dereferenced by the checks; the driver passes fake addresses.  It exits 0
// when it ran to the end; the sanitizers abort it on the first finding.
// Built and run by tests/test_sanitizers.py.
#include <stdint.h>
#include <stdio.h>

#include <limits>
#include <vector>

#include "validate.h"

using namespace bqd;

namespace {

const int64_t kBig = std::numeric_limits<int64_t>::max();
const int64_t kSmall = std::numeric_limits<int64_t>::min();
const int64_t kSizes[] = {kSmall, -1, 0, 1, 3, 16, 255, 256, 4096, (int64_t)1 << 29,
                          (int64_t)1 << 31, (int64_t)1 << 40, kBig - 1, kBig};

template <class T>
T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }

long checks = 0;
long accepted = 0;

void note(int64_t rc) {
  ++checks;
  if (rc == 0) ++accepted;
}

bqd_cq_matrix make_cq(int64_t output, int64_t input, int64_t padded, int64_t group, int64_t bits,
                      int64_t row_bytes) {
  bqd_cq_matrix m;
  m.output = output;
  m.input = input;
  m.input_padded = padded;
  m.group = group;
  m.bits = bits;
  m.row_bytes = row_bytes;
  m.packed = fake<const uint8_t>((uintptr_t)1 << 32);
  m.norms = fake<const uint16_t>((uintptr_t)2 << 32);
  m.codebook = fake<const float>((uintptr_t)3 << 32);
  return m;
}

}  // namespace

int main() {
  float* P = fake<float>((uintptr_t)4 << 32);
  float* Y = fake<float>((uintptr_t)5 << 32);
  float* X = fake<float>((uintptr_t)6 << 32);
  for (int64_t output : kSizes)
    for (int64_t padded : {(int64_t)-4, (int64_t)0, (int64_t)4, (int64_t)256, (int64_t)4096,
                           (int64_t)1 << 27, kBig})
      for (int64_t group : {(int64_t)0, (int64_t)1, (int64_t)3, (int64_t)64, (int64_t)1024,
                            (int64_t)2048})
        for (int64_t bits : {1, 2, 5, 6})
          for (int64_t row_bytes : {(int64_t)-1, (int64_t)0, (int64_t)64, (int64_t)2048, kBig}) {
            bqd_cq_matrix m = make_cq(output, padded > 1 ? padded - 1 : padded, padded, group, bits,
                                      row_bytes);
            note(check_cq_shape(&m));
            note(check_cq(&m));
            for (int64_t batch : {kSmall, (int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)8, kBig}) {
              note(check_prepare(&m, X, P, batch));
              for (int64_t rb : {kSmall, (int64_t)-1, (int64_t)0, (int64_t)5, kBig})
                for (int64_t rc : {kSmall, (int64_t)-1, (int64_t)0, (int64_t)1, kBig}) {
                  note(check_matvec(&m, P, Y, batch, rb, rc));
                  note(check_prepare_matvec(&m, X, P, Y, batch, rb, rc));
                }
            }
            for (int64_t n : kSizes) note(check_gather(&m, fake<const int32_t>((uintptr_t)7 << 32), n, Y));
            for (int64_t row : {kSmall, (int64_t)0, kBig}) note(check_unpack(&m, row, fake<uint8_t>(8)));
          }

  // several matrices: null and extreme row ranges, unequal shapes, overlaps
  std::vector<bqd_cq_matrix> ms(kMaxMulti + 1, make_cq(256, 200, 256, 64, 2, 64));
  std::vector<float*> ys(kMaxMulti + 1);
  for (size_t k = 0; k < ys.size(); ++k) ys[k] = fake<float>(((uintptr_t)16 + k) << 32);
  std::vector<int64_t> rb(kMaxMulti + 1), rc(kMaxMulti + 1), rbo(kMaxMulti + 1), rco(kMaxMulti + 1);
  for (int64_t n : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)3, kMaxMulti, kMaxMulti + 1})
    for (int64_t b : {kSmall, (int64_t)-1, (int64_t)0, (int64_t)255, kBig})
      for (int64_t c : {kSmall, (int64_t)-1, (int64_t)0, (int64_t)1, kBig})
        for (bool with_x : {false, true}) {
          for (auto& v : rb) v = b;
          for (auto& v : rc) v = c;
          note(check_matvec_multi(ms.data(), n, rb.data(), rc.data(), with_x, X, P, ys.data(),
                                  rbo.data(), rco.data()));
          note(check_matvec_multi(ms.data(), n, nullptr, rc.data(), with_x, X, P, ys.data(),
                                  rbo.data(), rco.data()));
          note(check_matvec_multi(ms.data(), n, rb.data(), nullptr, with_x, X, P, ys.data(),
                                  rbo.data(), rco.data()));
        }
  ms[1].output = kBig;
  note(check_matvec_multi(ms.data(), 2, nullptr, nullptr, false, nullptr, P, ys.data(), rbo.data(),
                          rco.data()));
  ms[1].output = kSmall;
  note(check_matvec_multi(ms.data(), 2, nullptr, nullptr, false, nullptr, P, ys.data(), rbo.data(),
                          rco.data()));

  const uint8_t* W = fake<const uint8_t>((uintptr_t)1 << 32);
  const uint8_t* S = fake<const uint8_t>((uintptr_t)2 << 32);
  for (int64_t R : kSizes)
    for (int64_t C : kSizes)
      for (int64_t batch : {(int64_t)-1, (int64_t)0, (int64_t)1, kBig}) {
        for (int64_t SR : {kSmall, (int64_t)0, (int64_t)1, (int64_t)4, kBig})
          for (int64_t SC : {kSmall, (int64_t)0, (int64_t)1, (int64_t)32, kBig})
            note(check_f8(W, R, C, S, SR, SC, X, Y, batch));
        for (int64_t G : {kSmall, (int64_t)0, (int64_t)1, (int64_t)16, kBig})
          note(check_i8(fake<const int8_t>((uintptr_t)1 << 32), R, C, S, G, X, Y, batch));
        note(check_kv_dot(fake<const int8_t>((uintptr_t)1 << 32), P, R, C, X, Y, batch));
        note(check_kv_quantize(X, R, C, fake<int8_t>((uintptr_t)9 << 32), Y));
        for (int64_t H : {(int64_t)0, (int64_t)1, (int64_t)2048, (int64_t)16384, (int64_t)32768, kBig})
          note(check_hadamard_mlp(X, R, H, P, P, P, P, nullptr, Y, batch));
      }
  for (int64_t n : kSizes) {
    note(check_decode(W, n, Y, 1));
    note(check_decode(W, n, Y, 2));
    note(check_read_stream(W, n, fake<uint32_t>((uintptr_t)5 << 32)));
    for (int64_t k : {kSmall, (int64_t)0, (int64_t)1, (int64_t)64, (int64_t)65, kBig}) {
      note(sample_workspace_need(n, k));
      for (int64_t ws : {kSmall, (int64_t)0, (int64_t)1 << 20, kBig})
        for (float t : {-1.0f, 0.0f, 0.7f, std::numeric_limits<float>::infinity(),
                        std::numeric_limits<float>::quiet_NaN()})
          note(check_sample_noalloc(X, n, k, t, fake<uint32_t>((uintptr_t)10 << 32),
                                    fake<int32_t>((uintptr_t)12 << 32),
                                    fake<int32_t>((uintptr_t)13 << 32),
                                    fake<float>((uintptr_t)14 << 32), ws)),
          note(check_sample(X, n, k, t, fake<uint32_t>((uintptr_t)10 << 32),
                            fake<void>((uintptr_t)11 << 32), ws, fake<int32_t>((uintptr_t)12 << 32),
                            fake<int32_t>((uintptr_t)13 << 32), fake<float>((uintptr_t)14 << 32)));
    }
  }
  printf("validate driver done: %ld checks, %ld accepted\n", checks, accepted);
  return accepted > 0 && accepted < checks ? 0 : 1;
}
