// Kernels of table row 2 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(2, Cfg2, Fast2)
