// Host check of the exact-KL Cactus functions of libspecverify (no GPU is
// touched).  Without arguments: reads "c delta" pairs (hexadecimal doubles) from
// stdin and prints "gamma steps" for each (gamma_star_kl), gamma as a hexadecimal
// double.  With the argument "div": reads "g c" pairs and prints the divergence
// (kl_divergence) of each.
#include "spec_verify.hip"
#include <cstdio>
#include <cstring>

int main(int argc, char** argv) {
  const bool div = argc > 1 && std::strcmp(argv[1], "div") == 0;
  double a = 0.0, b = 0.0;
  while (scanf("%la %la", &a, &b) == 2) {
    if (div) {
      printf("%a\n", specv::kl_divergence(a, b));
    } else {
      int steps = 0;
      const double g = specv::gamma_star_kl(a, b, &steps);
      printf("%a %d\n", g, steps);
    }
  }
  return 0;
}
