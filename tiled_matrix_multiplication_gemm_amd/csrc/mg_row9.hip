// Kernels of table row 9 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(9, Cfg9, Fast9)
