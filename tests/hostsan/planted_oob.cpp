// planted_oob.cpp -- a deliberate heap overflow and a signed overflow, built
// with the same sanitizer flags as the ABI layer, so that a CPU test can show
// the sanitized run reports such mistakes (host code only; never on a GPU).
#include <limits.h>

extern "C" int planted_heap_overflow(int i) {
  int* a = new int[4]();
  const int r = a[i];
  delete[] a;
  return r;
}

extern "C" int planted_signed_overflow(int x) { return x + INT_MAX; }
